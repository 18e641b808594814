"""CPU tests of the C ABI's host side: exported symbols, the tile classifier
against a brute-force dense mask, plan statistics, and layout validation.
No compute call is made: nothing here needs a GPU."""
import ctypes
import json
import os
import re

import numpy as np
import pytest

import oracle
from workloads import (CONFIGS, Layout, chunk_prompts, get_config, layout_from_chunks, prompt_draw, streaming_layout,
                       text_layout)

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "magi_attn.h")


def declared_functions():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"MAGI_API\s+[\w\s\*]*?\b(magi_attn_\w+)\s*\(", text)))


def test_library_exports_every_declared_symbol(built_lib):
    names = declared_functions()
    assert len(names) >= 9
    lib = ctypes.CDLL(built_lib)
    for n in names:
        assert hasattr(lib, n), n


def test_abi_version(built_lib):
    from block_causal_attention_flash_amd import magi_attn_abi_version
    hdr = open(os.path.join(ROOT, "include", "magi_attn.h")).read()
    declared = int(re.search(r"#define MAGI_ATTN_ABI_VERSION (\d+)", hdr).group(1))
    assert magi_attn_abi_version() == declared == 7


def brute_classes(layout, bm, bn, mask=None):
    mask = oracle.block_causal_mask(layout) if mask is None else mask
    tq, tk = mask.shape
    n_qt, n_kt = -(-tq // bm), -(-tk // bn)
    padded = np.zeros((n_qt * bm, n_kt * bn), dtype=bool)
    padded[:tq, :tk] = mask
    blocks = padded.reshape(n_qt, bm, n_kt, bn)
    rows_valid = np.zeros(n_qt * bm, dtype=bool)
    rows_valid[:tq] = True
    rv = rows_valid.reshape(n_qt, bm)
    cls = np.zeros((n_qt, n_kt), dtype=np.int8)
    for qt in range(n_qt):
        b = blocks[qt][rv[qt]]            # valid rows only
        allv = b.reshape(b.shape[0], n_kt, bn).all(axis=(0, 2))
        anyv = b.reshape(b.shape[0], n_kt, bn).any(axis=(0, 2))
        cls[qt] = np.where(allv, 2, np.where(anyv, 1, 0))
    return cls


def random_layout(rng):
    kind = rng.integers(0, 3)
    if kind == 0:
        vids = [[int(x) for x in rng.integers(1, 90, rng.integers(1, 5))] for _ in range(rng.integers(1, 4))]
        return layout_from_chunks(vids)
    if kind == 1:
        return streaming_layout(int(rng.integers(0, 4)), int(rng.integers(1, 4)), int(rng.integers(1, 70)))
    # separate q / kv offsets with some query-less chunks, several videos
    n = int(rng.integers(2, 8))
    qlen = [int(x) if rng.random() < 0.7 else 0 for x in rng.integers(1, 60, n)]
    klen = [int(x) for x in rng.integers(1, 60, n)]
    cuts = sorted(set([0, n] + [int(x) for x in rng.integers(1, n, rng.integers(0, 3))]))
    q = np.concatenate([[0], np.cumsum(qlen)]).tolist()
    kv = np.concatenate([[0], np.cumsum(klen)]).tolist()
    return Layout(tuple(q), tuple(kv), tuple(cuts))


@pytest.mark.parametrize("seed", range(40))
def test_classifier_matches_dense_mask(built_lib, seed):
    """Tile classes from the library against the oracle's dense mask, for
    random layouts with and without a KV range."""
    from block_causal_attention_flash_amd import magi_attn_classify_host
    rng = np.random.default_rng(seed)
    lay = random_layout(rng)
    if lay.t_q == 0:
        pytest.skip("no queries")
    for R, lg in ((0, 0), (int(rng.integers(1, 4)), 0), (0, 1), (int(rng.integers(1, 4)), 1)):
        lw = Layout(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, R, lg)
        mask = oracle.block_causal_mask(lw)
        if (mask.sum(axis=1) == 0).any():
            continue                          # a chunk with queries would see no key: rejected layout
        for bm, bn in ((64, 64), (128, 64), (32, 16), (7, 5)):
            got = magi_attn_classify_host(lw.q_offsets, lw.kv_offsets, lw.seq_chunks, bm=bm, bn=bn, kv_range=R,
                                          last_global=lg)
            np.testing.assert_array_equal(got, brute_classes(lw, bm, bn, mask))


def test_kv_range_stats_and_validation(built_lib):
    from block_causal_attention_flash_amd import MagiAttnError, magi_attn_plan_stats
    c = get_config("video480x832")
    st = magi_attn_plan_stats(c.layout.q_offsets, None, None, 48, 8, 128, "bf16", kv_range=5)
    assert st["unmasked_pairs"] == 9360 * 9360 * (1 + 2 + 3 + 4 + 5 * 12)
    assert st["executed_pairs"] / st["unmasked_pairs"] < 1.01
    full = magi_attn_plan_stats(c.layout.q_offsets, None, None, 48, 8, 128, "bf16", kv_range=16)
    assert full["unmasked_pairs"] == 9360 * 9360 * sum(range(1, 17))
    with pytest.raises(MagiAttnError) as e:
        magi_attn_plan_stats([0, 4, 8], None, None, 1, 1, 128, "bf16", kv_range=-1)
    assert e.value.status == 1
    # a chunk whose window holds no key: chunk 2 owns queries but no keys, R = 1
    with pytest.raises(MagiAttnError) as e:
        magi_attn_plan_stats([0, 4, 8, 12], [0, 4, 8, 8], None, 1, 1, 128, "bf16", kv_range=1)
    assert e.value.status == 1


def test_stats_match_mask_areas(built_lib):
    from block_causal_attention_flash_amd import magi_attn_plan_stats
    with open(os.path.join(ROOT, "tests", "golden", "unmasked_pairs.json")) as f:
        gold = json.load(f)["pairs_per_head"]
    for c in CONFIGS:
        lay = c.layout
        st = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, c.n_q_heads, c.n_kv_heads,
                                  c.head_dim, c.dtype)
        assert st["unmasked_pairs"] == gold[c.name]
        n_qt = -(-lay.t_q // st["tile_q"])
        n_kt = -(-lay.t_k // st["tile_kv"])
        assert st["full_pairs"] + st["boundary_pairs"] + st["empty_pairs"] == n_qt * n_kt
        # executed work covers the mask area with little waste
        assert gold[c.name] <= st["executed_pairs"] <= 1.05 * gold[c.name] + n_qt * st["tile_q"] * st["tile_kv"]
        groups = c.n_q_heads // c.n_kv_heads // st["heads_per_item"]
        assert st["n_items"] >= n_qt * c.n_kv_heads * groups


def test_stats_480p_tile_counts(built_lib):
    """16 chunks of 9360 tokens, 48 query heads on 8 KV heads: one work item
    covers 64 tokens of all 6 query heads of a KV head (384 rows), with
    32-key tiles; only tiles straddling a chunk end need the mask."""
    from block_causal_attention_flash_amd import magi_attn_plan_stats
    c = get_config("video480x832")
    st = magi_attn_plan_stats(c.layout.q_offsets, None, None, 48, 8, 128, "bf16")
    assert st["tile_q"] == 64 and st["tile_kv"] == 32 and st["heads_per_item"] == 6
    assert st["boundary_pairs"] < 0.01 * st["full_pairs"]
    assert st["executed_pairs"] / st["unmasked_pairs"] < 1.01


def test_bf16_head_dim_64_plans_like_128(built_lib):
    """head_dim 64 is accepted for bf16 and plans the same work items and tile
    lists as 128 (the tiling depends on the heads, not on head_dim)."""
    from block_causal_attention_flash_amd import magi_attn_plan_stats
    lay = get_config("streaming").layout
    for hq, hk in ((24, 8), (6, 2), (8, 1)):
        a = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, hq, hk, 64, "bf16")
        b = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, hq, hk, 128, "bf16")
        assert a == b


BAD = [
    (dict(q_offsets=[0, 4, 3]), 1),                                  # decreasing offsets
    (dict(q_offsets=[1, 4]), 1),                                     # not starting at 0
    (dict(q_offsets=[0, 4], seq_chunks=[0, 2]), 1),                  # seq_chunks beyond n_chunks
    (dict(q_offsets=[0, 4, 8], seq_chunks=[0, 1, 1, 2]), 1),         # empty video
    (dict(q_offsets=[0, 4], kv_offsets=[0, 0]), 1),                  # queries without keys
    (dict(q_offsets=[0, 4], n_q_heads=3, n_kv_heads=2), 1),          # heads not a multiple
    (dict(q_offsets=[0, 4], head_dim=96, dtype="bf16"), 2),          # unsupported head_dim
    (dict(q_offsets=[0, 4], head_dim=96, dtype="fp32"), 2),
    (dict(q_offsets=[0, 4], dtype=7), 1),                            # unknown dtype
]


@pytest.mark.parametrize("kw,status", BAD)
def test_invalid_layouts_are_rejected(built_lib, kw, status):
    from block_causal_attention_flash_amd import MagiAttnError, magi_attn_plan_create, magi_attn_plan_stats
    args = dict(n_q_heads=2, n_kv_heads=1, head_dim=128, dtype="bf16")
    args.update(kw)
    with pytest.raises(MagiAttnError) as e:
        magi_attn_plan_stats(**args)
    assert e.value.status == status and e.value.message
    # plan creation validates before any HIP call, so this is safe without a GPU
    with pytest.raises(MagiAttnError) as e:
        magi_attn_plan_create(**args)
    assert e.value.status == status


def test_streaming_cached_chunks_need_no_queries(built_lib):
    from block_causal_attention_flash_amd import magi_attn_plan_stats
    lay = get_config("streaming").layout
    st = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, 24, 8, 128, "bf16")
    assert st["unmasked_pairs"] == 1536 * 1536 * (17 + 18 + 19 + 20)
    assert st["boundary_pairs"] == 0


def random_text(rng, lay):
    n_prompts = int(rng.integers(0, 4))
    lens = [int(x) for x in rng.integers(1, 80, n_prompts)]
    choice = [None if (n_prompts == 0 or rng.random() < 0.3) else int(rng.integers(0, n_prompts))
              for _ in range(lay.n_chunks)]
    return chunk_prompts(choice, lens)


@pytest.mark.parametrize("seed", range(30))
def test_cross_classifier_matches_text_mask(built_lib, seed):
    """Tile classes of the cross-attention against the oracle's dense text
    mask, for random layouts and chunk-wise prompts (shared prompts, chunks
    without text, ragged prompt lengths)."""
    from block_causal_attention_flash_amd import magi_attn_cross_classify_host
    rng = np.random.default_rng(1000 + seed)
    lay = random_layout(rng)
    if lay.t_q == 0:
        pytest.skip("no queries")
    text = random_text(rng, lay)
    mask = oracle.text_mask(lay.q_offsets, text)
    for bm, bn in ((64, 32), (128, 32), (7, 5)):
        got = magi_attn_cross_classify_host(lay.q_offsets, text.begin, text.end, text.t_text, bm=bm, bn=bn,
                                            kv_offsets=lay.kv_offsets, seq_chunks=lay.seq_chunks)
        if text.t_text == 0:
            assert got.shape[1] == 0
            continue
        np.testing.assert_array_equal(got, brute_classes(lay, bm, bn, mask))


@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
def test_cross_and_parallel_stats(built_lib, name):
    """Pair counts of the workloads' cross-attention against the oracle's
    closed form; a parallel plan's counts are the sums of its two attentions
    and it holds every work item of both."""
    from block_causal_attention_flash_amd import magi_attn_cross_plan_stats, magi_attn_plan_stats
    c = get_config(name)
    lay, text = c.layout, text_layout(c)
    args = (lay.q_offsets, text.begin, text.end, text.t_text, lay.kv_offsets, lay.seq_chunks, c.n_q_heads,
            c.n_kv_heads, c.head_dim, c.dtype)
    x = magi_attn_cross_plan_stats(*args)
    assert x["unmasked_pairs"] == oracle.text_pairs(lay.q_offsets, text)
    n_qt = -(-lay.t_q // x["tile_q"])
    assert x["full_pairs"] + x["boundary_pairs"] + x["empty_pairs"] == n_qt * -(-text.t_text // x["tile_kv"])
    s = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, c.n_q_heads, c.n_kv_heads, c.head_dim,
                             c.dtype)
    p = magi_attn_cross_plan_stats(*args, with_self=True)
    for k in ("unmasked_pairs", "full_pairs", "boundary_pairs", "empty_pairs", "executed_pairs"):
        assert p[k] == s[k] + x[k], k
    assert p["n_items"] >= max(s["n_items"], x["n_items"])


TEXT_BAD = [
    (dict(text_begin=[0, 0], text_end=[0, 5], t_text=4), 1),          # end beyond t_text
    (dict(text_begin=[3, 0], text_end=[2, 0], t_text=4), 1),          # begin after end
    (dict(text_begin=[-1, 0], text_end=[0, 0], t_text=4), 1),         # negative begin
    (dict(text_begin=[0, 0], text_end=[0, 0], t_text=-1), 1),         # negative t_text
    (dict(text_begin=[0, 0], text_end=[0, 0], t_text=1 << 30), 2),    # text K/V of 2 GiB or more
]


@pytest.mark.parametrize("kw,status", TEXT_BAD)
def test_invalid_text_is_rejected(built_lib, kw, status):
    from block_causal_attention_flash_amd import (MagiAttnError, magi_attn_cross_plan_create,
                                                  magi_attn_cross_plan_stats, magi_attn_cross_train_plan_create,
                                                  magi_attn_parallel_plan_create)
    args = dict(q_offsets=[0, 4, 8], n_q_heads=2, n_kv_heads=1, head_dim=128, dtype="bf16")
    args.update(kw)
    for fn in (magi_attn_cross_plan_stats, magi_attn_cross_plan_create, magi_attn_parallel_plan_create,
               magi_attn_cross_train_plan_create):
        with pytest.raises(MagiAttnError) as e:
            fn(**args)
        assert e.value.status == status and e.value.message


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_cross_training_plan_limits_a_text_token_to_two_runs_of_rows(built_lib, dtype):
    """The backward keeps two token ranges per text key. Chunks 0, 2 and 4
    share one prompt with chunks of other prompts between them: three runs of
    rows, refused before any HIP call. (Two runs pass this check and go on to
    allocate the plan, which needs a GPU.)"""
    from block_causal_attention_flash_amd import MagiAttnError, magi_attn_cross_train_plan_create
    with pytest.raises(MagiAttnError) as e:
        magi_attn_cross_train_plan_create([0, 4, 8, 12, 16, 20], [0, 5, 0, 5, 0], [5, 9, 5, 9, 5], 9,
                                          n_q_heads=2, n_kv_heads=1, head_dim=128, dtype=dtype)
    assert e.value.status == 2 and "two" in e.value.message


def test_parallel_plan_size_limit(built_lib):
    """Video and text keys together are limited to 2 GiB of tile images
    (bf16): each alone fits, the two together do not."""
    from block_causal_attention_flash_amd import MagiAttnError, magi_attn_cross_plan_stats
    tk = 7 * (1 << 20) // 8                        # 0.875 Mi keys x 8 heads x 256 B = 1.75 GiB
    args = ([0, 16, tk], [0, 0], [0, tk // 4], tk // 4, None, None, 8, 8, 128, "bf16")
    magi_attn_cross_plan_stats(*args)                          # the text alone: 0.44 GiB
    with pytest.raises(MagiAttnError) as e:
        magi_attn_cross_plan_stats(*args, with_self=True)
    assert e.value.status == 2


def test_prompt_draw_structure():
    """The workload text recipe: clean chunks carry no text, cache chunks
    carry none, runs of chunks share one prompt."""
    lay = layout_from_chunks([[5] * 7, [3] * 2, [4]])
    t = prompt_draw(lay, 1, 3, seed=0, lo=10, hi=12)
    ranges = list(zip(t.begin, t.end))
    assert ranges[0] == (0, 0) and ranges[7] == (0, 0) and ranges[9] == (0, 0)
    assert ranges[1] == ranges[2] == ranges[3] and ranges[4] == ranges[5] == ranges[6] and ranges[1] != ranges[4]
    assert all(10 <= e - b <= 12 for b, e in ranges if e > b)
    assert t.t_text == max(t.end)
    st = prompt_draw(streaming_layout(3, 2, 4), 0, 1, seed=1)
    assert all(b == e for b, e in zip(st.begin[:3], st.end[:3]))


@pytest.mark.parametrize("seed", range(30))
def test_key_classifier_matches_transposed_mask(built_lib, seed):
    """The backward's (key block, token tile) classes against the transpose
    of the oracle's dense mask, for random layouts with and without a KV
    range."""
    from block_causal_attention_flash_amd import magi_attn_key_classify_host
    rng = np.random.default_rng(2000 + seed)
    lay = random_layout(rng)
    if lay.t_q == 0:
        pytest.skip("no queries")
    for R, lg in ((0, 0), (int(rng.integers(1, 4)), 0), (0, 1), (int(rng.integers(1, 4)), 1)):
        lw = Layout(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, R, lg)
        mask = oracle.block_causal_mask(lw)
        if (mask.sum(axis=1) == 0).any() and lw.t_q:
            continue                          # a chunk with queries would see no key: rejected layout
        for bk, bt in ((128, 32), (64, 32), (7, 5)):
            got = magi_attn_key_classify_host(lw.q_offsets, lw.kv_offsets, lw.seq_chunks, bk=bk, bt=bt, kv_range=R,
                                              last_global=lg)
            np.testing.assert_array_equal(got, brute_classes(lw, bk, bt, mask.T.copy()))


def test_last_global_stats(built_lib):
    """packed8 with its last video as a global block: the mask area in closed
    form (the other videos' block-causal area plus the global rows times T_k)."""
    from block_causal_attention_flash_amd import MagiAttnError, magi_attn_plan_stats
    c = get_config("packed8")
    lay = c.layout
    plain = magi_attn_plan_stats(lay.q_offsets, None, lay.seq_chunks, 32, 8, 128, "bf16")
    st = magi_attn_plan_stats(lay.q_offsets, None, lay.seq_chunks, 32, 8, 128, "bf16", last_global=1)
    g0 = lay.q_offsets[lay.seq_chunks[-2]]
    g_own = sum((lay.q_offsets[cc + 1] - lay.q_offsets[cc]) * (lay.q_offsets[cc + 1] - g0)
                for cc in range(lay.seq_chunks[-2], lay.n_chunks))
    assert st["unmasked_pairs"] == plain["unmasked_pairs"] - g_own + (lay.t_q - g0) * lay.t_q
    with pytest.raises(MagiAttnError):
        magi_attn_plan_stats([0, 4], None, None, 1, 1, 128, "bf16", last_global=2)


def test_split_piece_count_fills_whole_rounds(built_lib):
    """Split-KV piece counts (bf16). The streaming window has 384 whole items
    (128-token query tiles x 8 KV heads x 1 head group), under 2 per compute
    unit: with one item per CU at a time, 2 pieces per item make 768 pieces in
    3 full rounds of 256, where 3 pieces would take 4.5 rounds. Layouts with at
    least 512 items stay whole; a layout of 4 items is cut as finely as the
    64-tile minimum allows."""
    from block_causal_attention_flash_amd import magi_attn_plan_stats
    c = get_config("streaming")
    lay = c.layout
    st = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, c.n_q_heads, c.n_kv_heads, c.head_dim,
                              c.dtype)
    whole = -(-lay.t_q // st["tile_q"]) * c.n_kv_heads * (c.n_q_heads // c.n_kv_heads // st["heads_per_item"])
    assert whole == 384
    assert st["n_items"] == 2 * whole
    for name in ("video256x2", "video480x832"):
        c = get_config(name)
        lay = c.layout
        st = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, c.n_q_heads, c.n_kv_heads,
                                  c.head_dim, c.dtype)
        n_qt = -(-lay.t_q // st["tile_q"])
        assert st["n_items"] == n_qt * c.n_kv_heads * (c.n_q_heads // c.n_kv_heads // st["heads_per_item"]), name
    # 2 query tiles x 2 KV heads, each with 384 key tiles: 6 pieces of 64 tiles
    kv = [512 * i for i in range(17)] + [8192 + 2048, 8192 + 4096]
    q = [0] * 17 + [96, 192]
    st = magi_attn_plan_stats(q, kv, [0, 18], 6, 2, 128, "bf16")
    assert st["n_items"] >= 4 * 6


def test_plain_c_client_of_the_host_calls(built_lib, tmp_path):
    """The header compiles as strict C99 and a C program linked against the
    library gets the documented answers from the host-only calls (planning
    statistics, the tile classifier, the error path)."""
    import shutil
    import subprocess
    gcc = shutil.which("gcc")
    if gcc is None:
        pytest.skip("gcc not found")
    exe = tmp_path / "abi_host"
    libdir = os.path.dirname(built_lib)
    cmd = [gcc, "-std=c99", "-Wall", "-Wextra", "-pedantic", "-Werror", "-I", os.path.join(ROOT, "include"),
           os.path.join(ROOT, "tests", "c", "abi_host.c"), "-L", libdir, "-lmagi_attn", f"-Wl,-rpath,{libdir}",
           "-o", str(exe)]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr
    r = subprocess.run([str(exe)], capture_output=True, text=True, timeout=60)
    assert r.returncode == 0 and r.stdout.strip() == "ok", r.stdout + r.stderr


def test_tile_lists_past_int32_are_refused(built_lib):
    """One chunk of 8,388,000 tokens with one head passes the tensor limits
    (K is just under 2 GiB) but its tile lists would hold 5.7e9 entries,
    past the kernels' int32 indices: refused before any list is built."""
    from block_causal_attention_flash_amd import MagiAttnError, magi_attn_plan_stats
    with pytest.raises(MagiAttnError) as e:
        magi_attn_plan_stats([0, 8388000], None, None, 1, 1, 128, "bf16")
    assert e.value.status == 2 and "2^31" in e.value.message


def test_query_stream_length_limit(built_lib):
    """Query streams of 2^26 tokens or more are refused: int32 token indices
    keep their headroom and the per-row host tables stay below 512 MiB."""
    from block_causal_attention_flash_amd import MagiAttnError, magi_attn_plan_stats
    with pytest.raises(MagiAttnError) as e:
        magi_attn_plan_stats([0, 1 << 26], [0, 64], None, 1, 1, 128, "fp32")
    assert e.value.status == 2
