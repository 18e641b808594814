"""Pins of the fp64 oracle against facts that do not come from the oracle itself.

Each pin is chosen so that a plausible slip in the oracle fails it:
  * RMSNorm vs torch's rms_norm library routine (wrong axis, dropped eps or gain);
  * special layouts that reduce to library attention (torch SDPA in fp64):
      one chunk -> full bidirectional, size-1 chunks -> token-causal,
      one chunk per video -> varlen full, size-1 chunks per video -> varlen causal,
      cached chunks without queries -> full attention over the key prefix;
    these catch a wrong mask inequality, a wrong scale, a wrong GQA mapping;
  * pure-Python brute-force loops (math.exp / math.fsum) on tiny inputs;
  * causality: re-drawing later chunks / other videos leaves rows bitwise equal;
  * softmax rows sum to one, masked probabilities are exactly zero;
  * closed forms: identical keys give uniform weights over the allowed range
    [video start, end of own chunk), computed from the offsets by hand;
  * the log-sum-exp merge identity over a split key set.
The mask semantics come from the MAGI-1 pages: paperlayer §2 / Figure 1 and
paper-notes §2 / Figure 1 (bidirectional in a chunk, causal across chunks),
paper-notes Figure 15 (varlen block-causal: no cross-video attention),
paperlayer §2.4.4 (KV cache); the FLOP area from paperlayer §B.2.1.
"""
import json
import math
import os

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import dense as oracle_mod
from workloads import Layout, get_config, layout_from_chunks, make_inputs, streaming_layout

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _t64(x):
    return x.detach().to(torch.float64)


def lib_attention(q, k, v, qg, kg, eps, scale, causal=False):
    """Library reference: torch rms_norm + SDPA in fp64, KV heads repeated
    (contiguous groups).  q: [T,Hq,d] -> out [T,Hq,d]."""
    q, k, v = _t64(q), _t64(k), _t64(v)
    d = q.shape[-1]
    qh = F.rms_norm(q, (d,), _t64(qg), eps)
    kh = F.rms_norm(k, (d,), _t64(kg), eps)
    group = q.shape[1] // k.shape[1]
    kh = kh.repeat_interleave(group, dim=1)
    vv = v.repeat_interleave(group, dim=1)
    o = F.scaled_dot_product_attention(qh.transpose(0, 1)[None], kh.transpose(0, 1)[None].contiguous(),
                                       vv.transpose(0, 1)[None].contiguous(), is_causal=causal, scale=scale)
    return o[0].transpose(0, 1).numpy()


def small_inputs(layout, hq=4, hk=2, d=16, seed=0, gains="uniform"):
    return make_inputs(layout, hq, hk, d, "fp32", gains, seed)


# ----------------------------------------------------------------------------- pins

def check_rms(fn=oracle.rms_norm):
    rng = np.random.default_rng(0)
    x = rng.standard_normal((7, 3, 32))
    g = rng.uniform(0.5, 1.5, 32)
    for eps in (1e-6, 0.5):
        ref = F.rms_norm(torch.from_numpy(x), (32,), torch.from_numpy(g), eps).numpy()
        got = fn(x, g, eps)
        if not np.allclose(got, ref, rtol=1e-13, atol=1e-13):
            return False
    return True


def check_single_chunk(fn=oracle.attention):
    lay = layout_from_chunks([[37]])
    inp = small_inputs(lay, 6, 2, 16, seed=1)
    scale = 0.37
    out, _ = fn(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, scale, lay)
    ref = lib_attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, scale)
    return np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def check_token_causal(fn=oracle.attention):
    lay = layout_from_chunks([[1] * 23])
    inp = small_inputs(lay, 4, 2, 16, seed=2)
    out, _ = fn(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.25, lay)
    ref = lib_attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.25, causal=True)
    return np.allclose(out, ref, rtol=1e-12, atol=1e-12)


def check_varlen(fn=oracle.attention, causal=False):
    lens = [11, 5, 17]
    vids = [[1] * n for n in lens] if causal else [[n] for n in lens]
    lay = layout_from_chunks(vids)
    inp = small_inputs(lay, 4, 1, 8, seed=3)
    out, _ = fn(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.5, lay)
    o = 0
    for n in lens:
        sl = slice(o, o + n)
        ref = lib_attention(inp["q"][sl], inp["k"][sl], inp["v"][sl], inp["q_gain"], inp["k_gain"], 1e-6, 0.5,
                            causal=causal)
        if not np.allclose(out[sl], ref, rtol=1e-12, atol=1e-12):
            return False
        o += n
    return True


def check_streaming_prefix(fn=oracle.attention):
    lay = streaming_layout(3, 2, 6)          # 3 cached chunks, 2 active, 6 tokens each
    inp = small_inputs(lay, 4, 2, 8, seed=4)
    out, _ = fn(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    for a in range(2):
        sl = slice(6 * a, 6 * a + 6)
        kend = 6 * (3 + a + 1)
        ref = lib_attention(inp["q"][sl], inp["k"][:kend], inp["v"][:kend], inp["q_gain"], inp["k_gain"],
                            1e-6, 0.3)
        if not np.allclose(out[sl], ref, rtol=1e-12, atol=1e-12):
            return False
    return True


def allowed_range(layout, i):
    """[video start, end of own chunk) in key tokens, from the offsets; with a
    KV range R the start is that of chunk c - R + 1 when it is later."""
    c = max(cc for cc in range(len(layout.q_offsets) - 1) if layout.q_offsets[cc] <= i < layout.q_offsets[cc + 1])
    s = max(ss for ss in range(len(layout.seq_chunks) - 1) if layout.seq_chunks[ss] <= c)
    first = layout.seq_chunks[s]
    if layout.kv_range > 0:
        first = max(first, c - layout.kv_range + 1)
    return layout.kv_offsets[first], layout.kv_offsets[c + 1]


def check_identical_keys(fn=oracle.attention, layout=None):
    lay = layout or Layout((0, 0, 0, 5, 9, 9, 16, 20), (0, 4, 7, 12, 15, 18, 22, 26), (0, 4, 7))
    tq, tk = lay.t_q, lay.t_k
    rng = np.random.default_rng(5)
    hq, hk, d = 4, 2, 8
    q = rng.standard_normal((tq, hq, d))
    krow = rng.standard_normal((1, hk, d))
    k = np.repeat(krow, tk, axis=0)
    v = rng.standard_normal((tk, hk, d))
    qg, kg = rng.uniform(0.5, 1.5, d), rng.uniform(0.5, 1.5, d)
    scale = 0.41
    out, lse = fn(q, k, v, qg, kg, 1e-6, scale, lay)
    qh = F.rms_norm(torch.from_numpy(q), (d,), torch.from_numpy(qg), 1e-6).numpy()
    kh = F.rms_norm(torch.from_numpy(krow), (d,), torch.from_numpy(kg), 1e-6).numpy()[0]
    for i in range(tq):
        lo, hi = allowed_range(lay, i)
        for h in range(hq):
            g = h // (hq // hk)
            if not np.allclose(out[i, h], v[lo:hi, g].mean(axis=0), rtol=1e-12, atol=1e-12):
                return False
            s = scale * float(np.dot(qh[i, h], kh[g]))
            if abs(lse[h, i] - (s + math.log(hi - lo))) > 1e-12:
                return False
    return True


def windowed(layout, R):
    return Layout(layout.q_offsets, layout.kv_offsets, layout.seq_chunks, R)


def check_window_wide_is_block_causal(fn=oracle.attention):
    """A KV range of at least the number of chunks changes nothing."""
    lay = layout_from_chunks([[5, 7, 3], [4, 6]])
    inp = small_inputs(lay, 4, 2, 8, seed=15)
    args = (inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3)
    o0, l0 = fn(*args, lay)
    o1, l1 = fn(*args, windowed(lay, 3))
    o2, l2 = fn(*args, windowed(lay, 50))
    return all(np.array_equal(a, b) for a, b in ((o0, o1), (l0, l1), (o0, o2), (l0, l2)))


def check_window_slices(R, fn=oracle.attention):
    """KV range R: the rows of chunk c are full attention (library SDPA) over
    the keys of chunks max(first, c - R + 1) .. c of their video."""
    lay = windowed(layout_from_chunks([[5, 7, 3, 6], [4, 6]]), R)
    inp = small_inputs(lay, 4, 2, 8, seed=16)
    out, _ = fn(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    for s in range(lay.n_seqs):
        c0, c1 = lay.seq_chunks[s], lay.seq_chunks[s + 1]
        for c in range(c0, c1):
            rows = slice(lay.q_offsets[c], lay.q_offsets[c + 1])
            keys = slice(lay.kv_offsets[max(c0, c - R + 1)], lay.kv_offsets[c + 1])
            ref = lib_attention(inp["q"][rows], inp["k"][keys], inp["v"][keys], inp["q_gain"], inp["k_gain"],
                                1e-6, 0.3)
            if not np.allclose(out[rows], ref, rtol=1e-12, atol=1e-12):
                return False
    return True


# ----------------------------------------------------------------------------- tests

def test_rms_norm_matches_library():
    assert check_rms()


def test_single_chunk_is_full_attention():
    assert check_single_chunk()


def test_size_one_chunks_are_token_causal():
    assert check_token_causal()


def test_one_chunk_per_video_is_varlen_full():
    assert check_varlen(causal=False)


def test_size_one_chunks_per_video_is_varlen_causal():
    assert check_varlen(causal=True)


def test_streaming_window_is_prefix_attention():
    assert check_streaming_prefix()


def test_identical_keys_closed_form_mixed_layout():
    assert check_identical_keys()


@pytest.mark.parametrize("name", ["streaming", "packed8"])
def test_identical_keys_closed_form_config_geometry(name):
    """The closed form on the chunk geometry of the streaming and packed configs,
    shrunk by a constant factor so the dense oracle stays small."""
    lay = get_config(name).layout
    f = 128
    shrink = Layout(tuple(x // f for x in lay.q_offsets), tuple(x // f for x in lay.kv_offsets), lay.seq_chunks)
    assert all(b - a >= 0 for a, b in zip(shrink.q_offsets, shrink.q_offsets[1:]))
    assert check_identical_keys(layout=shrink)


def test_brute_force_loops_tiny_config():
    cfg = get_config("tiny")
    inp = make_inputs(cfg.layout, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype, cfg.gain_kind, cfg.seed)
    args = (inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], cfg.eps, cfg.scale, cfg.layout)
    o1, l1 = oracle.attention(*args)
    o2, l2 = oracle.attention_loops(*args)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


def test_brute_force_loops_packed_streaming():
    lay = Layout((0, 0, 3, 7, 7, 12), (0, 2, 5, 8, 11, 14), (0, 3, 5))
    inp = small_inputs(lay, 4, 2, 8, seed=6)
    args = (inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    o1, l1 = oracle.attention(*args)
    o2, l2 = oracle.attention_loops(*args)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


def test_later_chunks_do_not_leak():
    """Re-drawing K/V of every chunk after chunk i leaves chunk i bitwise equal."""
    lay = layout_from_chunks([[5, 7, 3, 6]])
    inp = small_inputs(lay, 4, 2, 8, seed=7)
    base, base_lse = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    rng = np.random.default_rng(8)
    for c in range(3):
        k = inp["k"].clone()
        v = inp["v"].clone()
        start = lay.kv_offsets[c + 1]
        k[start:] = torch.from_numpy(rng.standard_normal(k[start:].shape).astype(np.float32))
        v[start:] = torch.from_numpy(rng.standard_normal(v[start:].shape).astype(np.float32))
        o, l_ = oracle.attention(inp["q"], k, v, inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
        rows = slice(0, lay.q_offsets[c + 1])
        assert np.array_equal(o[rows], base[rows])
        assert np.array_equal(l_[:, rows], base_lse[:, rows])
        assert not np.array_equal(o[lay.q_offsets[c + 1]:], base[lay.q_offsets[c + 1]:])


def test_other_videos_do_not_leak():
    lay = layout_from_chunks([[4, 4], [3, 5, 2], [6]])
    inp = small_inputs(lay, 2, 1, 8, seed=9)
    base, _ = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    k = inp["k"].clone()
    v = inp["v"].clone()
    a, b = lay.kv_offsets[lay.seq_chunks[1]], lay.kv_offsets[lay.seq_chunks[2]]
    k[a:b] *= -2.0
    v[a:b] += 1.0
    o, _ = oracle.attention(inp["q"], k, v, inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    assert np.array_equal(o[:a], base[:a]) and np.array_equal(o[b:], base[b:])
    assert not np.array_equal(o[a:b], base[a:b])


def test_softmax_rows_sum_to_one_and_masked_are_zero():
    lay = Layout((0, 0, 4, 9, 9, 13), (0, 3, 6, 9, 12, 15), (0, 3, 5))
    inp = small_inputs(lay, 4, 2, 8, seed=10)
    p = oracle.attention_probs(inp["q"], inp["k"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    assert np.max(np.abs(p.sum(axis=-1) - 1.0)) <= 1e-12
    mask = oracle.block_causal_mask(lay)
    assert np.all(p[:, ~mask] == 0.0)
    assert np.all(p[:, mask] > 0.0)


def test_constant_values_pass_through():
    lay = layout_from_chunks([[3, 4], [5]])
    inp = small_inputs(lay, 2, 1, 8, seed=11)
    vconst = torch.full_like(inp["v"], 0.75)
    o, _ = oracle.attention(inp["q"], inp["k"], vconst, inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    assert np.max(np.abs(o - 0.75)) <= 1e-14


def test_query_scaling_invariance_without_eps():
    lay = layout_from_chunks([[4, 6]])
    inp = small_inputs(lay, 2, 1, 8, seed=12)
    o1, l1 = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 0.0, 0.3, lay)
    q64, k64 = inp["q"].double(), inp["k"].double()
    o2, l2 = oracle.attention(q64 * 3.5, k64 * 0.2, inp["v"], inp["q_gain"], inp["k_gain"], 0.0, 0.3, lay)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12) and np.allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_gqa_equals_mha_with_repeated_kv():
    lay = layout_from_chunks([[5, 3]])
    inp = small_inputs(lay, 6, 2, 8, seed=13)
    o1, l1 = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    k = inp["k"].repeat_interleave(3, dim=1)
    v = inp["v"].repeat_interleave(3, dim=1)
    o2, l2 = oracle.attention(inp["q"], k, v, inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)


def test_lse_merge_identity():
    """Queries Q attend to keys A (layout 1), to keys B (layout 2) and to A u B
    (layout 3); the third result is the lse-weighted merge of the first two."""
    na, nb, nq = 6, 5, 4
    rng = np.random.default_rng(14)
    d = 8
    q = rng.standard_normal((nq, 2, d))
    ka, kb = rng.standard_normal((na, 1, d)), rng.standard_normal((nb, 1, d))
    va, vb = rng.standard_normal((na, 1, d)), rng.standard_normal((nb, 1, d))
    g = np.ones(d)
    la = Layout((0, 0, nq), (0, 0, na), (0, 2))            # queries in chunk 1 see all of A
    lb = Layout((0, 0, nq), (0, 0, nb), (0, 2))
    lab = Layout((0, 0, nq), (0, na, na + nb), (0, 2))      # chunk 0 holds A, chunk 1 holds B
    oa, sa = oracle.attention(q, ka, va, g, g, 1e-6, 0.3, la)
    ob, sb = oracle.attention(q, kb, vb, g, g, 1e-6, 0.3, lb)
    oab, sab = oracle.attention(q, np.concatenate([ka, kb]), np.concatenate([va, vb]), g, g, 1e-6, 0.3, lab)
    lse = np.logaddexp(sa, sb)
    wa = np.exp(sa - lse).T[:, :, None]
    wb = np.exp(sb - lse).T[:, :, None]
    assert np.allclose(sab, lse, rtol=0, atol=1e-12)
    assert np.allclose(oab, wa * oa + wb * ob, rtol=0, atol=1e-12)


def test_unmasked_pairs_closed_forms():
    """Mask area per head: sum over query chunks of (own tokens) x (keys from the
    video's start to the end of the chunk) -- checked against hand formulas."""
    assert oracle.unmasked_pairs(get_config("tiny").layout) == 64 * 64 * (1 + 2 + 3)
    assert oracle.unmasked_pairs(streaming_layout(2, 3, 7)) == 7 * 7 * (3 + 4 + 5)
    assert oracle.unmasked_pairs(layout_from_chunks([[3, 3], [5]])) == 9 + 18 + 25
    with open(os.path.join(GOLDEN, "unmasked_pairs.json")) as f:
        gold = json.load(f)["pairs_per_head"]
    assert gold["video480x832"] == 9360 * 9360 * sum(range(1, 17))
    assert gold["video256x2"] == 2 * 1536 * 1536 * (1 + 2 + 3 + 4)
    assert gold["streaming"] == 1536 * 1536 * (17 + 18 + 19 + 20)
    packed = get_config("packed8").layout
    expect = 0
    for s in range(packed.n_seqs):
        c0, c1 = packed.seq_chunks[s], packed.seq_chunks[s + 1]
        size = packed.q_offsets[c0 + 1] - packed.q_offsets[c0]
        n = c1 - c0
        expect += size * size * n * (n + 1) // 2
    assert gold["packed8"] == expect
    for name in ("tiny", "video256x2", "streaming"):
        assert gold[name] == oracle.unmasked_pairs(get_config(name).layout)


def test_kv_range_wide_is_block_causal():
    assert check_window_wide_is_block_causal()


@pytest.mark.parametrize("R", [1, 2, 3])
def test_kv_range_is_full_attention_over_the_last_chunks(R):
    assert check_window_slices(R)


def test_kv_range_brute_force_loops():
    lay = Layout((0, 0, 3, 7, 7, 12, 14), (0, 2, 5, 8, 11, 14, 17), (0, 4, 6), 2)
    inp = small_inputs(lay, 4, 2, 8, seed=17)
    args = (inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    o1, l1 = oracle.attention(*args)
    o2, l2 = oracle.attention_loops(*args)
    assert np.max(np.abs(o1 - o2)) <= 1e-12
    assert np.max(np.abs(l1 - l2)) <= 1e-12


@pytest.mark.parametrize("R", [1, 2, 4])
def test_kv_range_identical_keys_closed_form(R):
    lay = Layout((0, 0, 0, 5, 9, 9, 16, 20), (0, 4, 7, 12, 15, 18, 22, 26), (0, 4, 7), R)
    assert check_identical_keys(layout=lay)


def test_kv_range_unmasked_pairs_closed_form():
    lay = windowed(layout_from_chunks([[3, 4, 5, 6]]), 2)
    assert oracle.unmasked_pairs(lay) == 3 * 3 + 4 * (3 + 4) + 5 * (4 + 5) + 6 * (5 + 6)
    # the 16-chunk geometry of the 480x832 video with a KV range of 5, at 90 tokens per chunk
    assert oracle.unmasked_pairs(windowed(layout_from_chunks([[90] * 16]), 5)) == 90 * 90 * (1 + 2 + 3 + 4 + 5 * 12)


def _window_off_by_one(layout, rows=None):
    """Mutant: a KV range R admits R + 1 chunks."""
    m = _orig_mask(Layout(layout.q_offsets, layout.kv_offsets, layout.seq_chunks), rows)
    tq, tk = int(layout.q_offsets[-1]), int(layout.kv_offsets[-1])
    qc = oracle.token_chunk_ids(layout.q_offsets, tq)
    kc = oracle.token_chunk_ids(layout.kv_offsets, tk)
    if rows is not None:
        qc = qc[np.asarray(rows)]
    if layout.kv_range > 0:
        m &= kc[None, :] >= qc[:, None] - layout.kv_range
    return m


def test_planted_window_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(oracle_mod, "block_causal_mask", _window_off_by_one)
    assert not check_window_slices(2, oracle_mod.attention)


# ----------------------------------------------------------------------------- planted mistakes

def _mutant_mask_no_video(layout, rows=None):
    tq, tk = int(layout.q_offsets[-1]), int(layout.kv_offsets[-1])
    qc = oracle.token_chunk_ids(layout.q_offsets, tq)
    kc = oracle.token_chunk_ids(layout.kv_offsets, tk)
    if rows is not None:
        qc = qc[np.asarray(rows)]
    return kc[None, :] <= qc[:, None]


@pytest.mark.parametrize("mutant,checks", [
    ("mask_strict", ["single_chunk", "identical_keys"]),
    ("mask_no_video", ["varlen_full", "identical_keys"]),
    ("rms_no_eps", ["rms"]),
    ("gqa_modulo", ["single_chunk"]),
    ("lse_log2", ["identical_keys"]),
])
def test_planted_mistakes_are_caught(monkeypatch, mutant, checks):
    """Each mistake planted in the oracle (on the CPU) makes some pin fail."""
    if mutant == "mask_strict":
        monkeypatch.setattr(oracle_mod, "block_causal_mask",
                            lambda lay, rows=None: _strict_mask(lay, rows))
    elif mutant == "mask_no_video":
        monkeypatch.setattr(oracle_mod, "block_causal_mask", _mutant_mask_no_video)
    elif mutant == "rms_no_eps":
        monkeypatch.setattr(oracle_mod, "rms_norm", lambda x, g, eps: _orig_rms(x, g, 0.0))
    elif mutant == "gqa_modulo":
        monkeypatch.setattr(oracle_mod, "attention", _gqa_modulo_attention)
    elif mutant == "lse_log2":
        monkeypatch.setattr(oracle_mod, "attention", _lse_log2_attention)
    results = {
        "single_chunk": lambda: check_single_chunk(oracle_mod.attention),
        "identical_keys": lambda: check_identical_keys(oracle_mod.attention),
        "varlen_full": lambda: check_varlen(oracle_mod.attention, causal=False),
        "rms": lambda: check_rms(lambda x, g, eps: oracle_mod.rms_norm(x, g, eps)),
    }
    assert any(not results[c]() for c in checks)


_orig_rms = oracle_mod.rms_norm
_orig_mask = oracle_mod.block_causal_mask
_orig_attention = oracle_mod.attention


def _strict_mask(layout, rows=None):
    """Mutant: a chunk does not see itself (strict inequality)."""
    tq, tk = int(layout.q_offsets[-1]), int(layout.kv_offsets[-1])
    qc = oracle.token_chunk_ids(layout.q_offsets, tq)
    kc = oracle.token_chunk_ids(layout.kv_offsets, tk)
    vid = oracle.chunk_video_ids(layout.seq_chunks, len(layout.q_offsets) - 1)
    if rows is not None:
        qc = qc[np.asarray(rows)]
    m = (vid[qc][:, None] == vid[kc][None, :]) & (kc[None, :] < qc[:, None])
    # keep every row non-empty so the mutant still returns finite numbers
    first = np.zeros_like(m)
    first[:, 0] = True
    return m | first


def _gqa_modulo_attention(q, k, v, qg, kg, eps, scale, layout, rows=None, row_block=256):
    """Mutant: query head h uses KV head h % H_kv (interleaved groups)."""
    q = oracle_mod._as_f64(q)
    k = oracle_mod._as_f64(k)
    v = oracle_mod._as_f64(v)
    hq, hk = q.shape[1], k.shape[1]
    perm = [h % hk for h in range(hq)]
    kk = k[:, perm, :]
    vv = v[:, perm, :]
    return _orig_attention(q, kk, vv, qg, kg, eps, scale, layout, rows, row_block)


def _lse_log2_attention(*args, **kw):
    """Mutant: log-sum-exp reported in base 2."""
    o, l = _orig_attention(*args, **kw)
    return o, l / math.log(2.0)


# ----------------------------------------------------------------------------- last global block

def global_case():
    base = layout_from_chunks([[7, 5, 9], [4, 6], [3, 8]])
    return Layout(base.q_offsets, base.kv_offsets, base.seq_chunks, 0, 1)


def check_global_rows(fn=oracle.attention):
    """The last video's queries (the global block) attend to every key of the
    stream: full attention over all keys (SDPA); every other row is as
    without the flag."""
    lay = global_case()
    inp = small_inputs(lay, 4, 2, 16, seed=31)
    out, lse = fn(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, lay)
    g0 = lay.q_offsets[lay.seq_chunks[-2]]
    ref = lib_attention(inp["q"][g0:], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3)
    plain = Layout(lay.q_offsets, lay.kv_offsets, lay.seq_chunks)
    o2, _ = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.3, plain)
    return np.allclose(out[g0:], ref, rtol=1e-12, atol=1e-12) and np.array_equal(out[:g0], o2[:g0])


def test_last_global_block_is_full_attention_over_the_stream():
    assert check_global_rows()


def test_last_global_block_brute_force_loops():
    lay = global_case()
    inp = small_inputs(lay, 4, 2, 8, seed=32)
    a = (inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.5, lay)
    o1, l1 = oracle.attention(*a)
    o2, l2 = oracle.attention_loops(*a)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12) and np.allclose(l1, l2, rtol=1e-12, atol=1e-12)


def test_last_global_block_mask_area():
    lay = global_case()
    plain = Layout(lay.q_offsets, lay.kv_offsets, lay.seq_chunks)
    g0 = lay.q_offsets[lay.seq_chunks[-2]]
    own = int(oracle.block_causal_mask(plain)[:g0].sum())
    assert oracle.unmasked_pairs(lay) == own + (lay.t_q - g0) * lay.t_k


def test_planted_global_mistake_is_caught(monkeypatch):
    """Mutant: the global flag is ignored (the last video stays block-causal)."""
    monkeypatch.setattr(oracle_mod, "block_causal_mask",
                        lambda lay, rows=None: _orig_mask(Layout(lay.q_offsets, lay.kv_offsets, lay.seq_chunks,
                                                                 lay.kv_range), rows))
    assert not check_global_rows(oracle_mod.attention)
