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
from workloads import CONFIGS, Layout, get_config, layout_from_chunks, streaming_layout

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
    assert magi_attn_abi_version() == declared == 2


def brute_classes(layout, bm, bn):
    mask = oracle.block_causal_mask(layout)
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
    for R in (0, int(rng.integers(1, 4))):
        lw = Layout(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, R)
        if R and any(lw.q_offsets[c + 1] > lw.q_offsets[c] and lw.kv_offsets[c + 1] == lw.kv_offsets[max(
                [s0 for s0 in lw.seq_chunks[:-1] if s0 <= c][-1], c - R + 1)] for c in range(lw.n_chunks)):
            continue                          # a chunk with queries would see no key: rejected layout
        for bm, bn in ((64, 64), (128, 64), (32, 16), (7, 5)):
            got = magi_attn_classify_host(lw.q_offsets, lw.kv_offsets, lw.seq_chunks, bm=bm, bn=bn, kv_range=R)
            np.testing.assert_array_equal(got, brute_classes(lw, bm, bn))


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


BAD = [
    (dict(q_offsets=[0, 4, 3]), 1),                                  # decreasing offsets
    (dict(q_offsets=[1, 4]), 1),                                     # not starting at 0
    (dict(q_offsets=[0, 4], seq_chunks=[0, 2]), 1),                  # seq_chunks beyond n_chunks
    (dict(q_offsets=[0, 4, 8], seq_chunks=[0, 1, 1, 2]), 1),         # empty video
    (dict(q_offsets=[0, 4], kv_offsets=[0, 0]), 1),                  # queries without keys
    (dict(q_offsets=[0, 4], n_q_heads=3, n_kv_heads=2), 1),          # heads not a multiple
    (dict(q_offsets=[0, 4], head_dim=64, dtype="bf16"), 2),          # unsupported head_dim for bf16
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
