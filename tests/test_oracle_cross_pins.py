"""Pins of the fp64 cross-attention oracle (oracle/cross.py) against facts that
do not come from the oracle itself.

  * each chunk's rows equal library attention (torch rms_norm + SDPA in fp64,
    no mask) over exactly that chunk's text slice; chunks without text give
    out 0 and lse -inf (catches a wrong range end, a normalised V, an
    un-normalised q, text leaking into clean chunks, a wrong GQA map);
  * pure-Python brute-force loops on tiny inputs;
  * locality: re-drawing text outside a chunk's range leaves its rows bitwise
    equal;
  * closed form: identical text keys give uniform weights over the range;
  * the pair count (the FLOP area) against the dense mask.
The operation comes from the MAGI-1 pages: paperlayer §2.2.2 and paper-notes
§3.2.2 (parallel self- and cross-attention with a shared query projection,
QK-Norm and GQA on both), paperlayer §2.2.3 (chunk-wise prompts) and
paper-notes §3.2.6 (clean chunks carry no text).
"""
import math

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import cross as cross_mod
from oracle import dense as dense_mod
from workloads import (chunk_prompts, get_config, layout_from_chunks, make_inputs, make_text_inputs,
                       streaming_layout, text_layout)


def _t64(x):
    return x.detach().to(torch.float64)


def lib_full_attention(q, k, v, qg, kg, eps, scale):
    """torch rms_norm + SDPA (fp64, no mask), KV heads repeated in contiguous
    groups. q [T,Hq,d], k/v [S,Hk,d] -> out [T,Hq,d], lse [Hq,T]."""
    q, k, v = _t64(q), _t64(k), _t64(v)
    d = q.shape[-1]
    qh = F.rms_norm(q, (d,), _t64(qg), eps)
    kh = F.rms_norm(k, (d,), _t64(kg), eps)
    group = q.shape[1] // k.shape[1]
    kh = kh.repeat_interleave(group, dim=1).transpose(0, 1).contiguous()
    vv = v.repeat_interleave(group, dim=1).transpose(0, 1).contiguous()
    o = F.scaled_dot_product_attention(qh.transpose(0, 1)[None], kh[None], vv[None], scale=scale)
    lse = torch.logsumexp(scale * qh.transpose(0, 1) @ kh.transpose(1, 2), dim=-1)
    return o[0].transpose(0, 1).numpy(), lse.numpy()


def case(lay, text, hq=4, hk=2, d=16, seed=0):
    inp = make_inputs(lay, hq, hk, d, "fp32", "uniform", seed)
    tx = make_text_inputs(text, hk, d, "fp32", "uniform", seed + 1)
    return inp, tx


def _mixed_case():
    # two videos; chunk 0 of each is clean; chunks 1-2 share a prompt; a
    # prompt shorter than a tile and one prompt used by two videos
    lay = layout_from_chunks([[9, 13, 7, 11], [5, 8]])
    text = chunk_prompts([None, 0, 0, 1, None, 1], [6, 19])
    return lay, text


def check_slices(fn=oracle.cross_attention, lay=None, text=None, hq=4, hk=2, scale=0.41):
    if lay is None:
        lay, text = _mixed_case()
    inp, tx = case(lay, text, hq, hk)
    out, lse = fn(inp["q"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, scale, lay.q_offsets, text)
    for c in range(lay.n_chunks):
        sl = slice(lay.q_offsets[c], lay.q_offsets[c + 1])
        b, e = text.begin[c], text.end[c]
        if b == e:
            if not (np.all(out[sl] == 0.0) and np.all(lse[:, sl] == -np.inf)):
                return False
            continue
        ro, rl = lib_full_attention(inp["q"][sl], tx["k_x"][b:e], tx["v_x"][b:e], tx["q_gain_x"], tx["k_gain_x"],
                                    1e-6, scale)
        if not (np.allclose(out[sl], ro, rtol=1e-12, atol=1e-12) and np.allclose(lse[:, sl], rl, rtol=1e-12,
                                                                                 atol=1e-12)):
            return False
    return True


def check_identical_keys(fn=oracle.cross_attention):
    lay, text = _mixed_case()
    inp, tx = case(lay, text)
    k = tx["k_x"].clone()
    k[:] = k[0:1]
    scale = 0.3
    out, lse = fn(inp["q"], k, tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, scale, lay.q_offsets, text)
    v = _t64(tx["v_x"]).numpy()
    qh = F.rms_norm(_t64(inp["q"]), (16,), _t64(tx["q_gain_x"]), 1e-6).numpy()
    kh = F.rms_norm(_t64(k[0]), (16,), _t64(tx["k_gain_x"]), 1e-6).numpy()
    for c in range(lay.n_chunks):
        b, e = text.begin[c], text.end[c]
        for i in range(lay.q_offsets[c], lay.q_offsets[c + 1]):
            for h in range(4):
                g = h // 2
                if b == e:
                    ok = np.all(out[i, h] == 0) and lse[h, i] == -np.inf
                else:
                    s = scale * float(qh[i, h] @ kh[g])
                    ok = (np.allclose(out[i, h], v[b:e, g].mean(axis=0), rtol=1e-12, atol=1e-12)
                          and abs(lse[h, i] - (s + math.log(e - b))) < 1e-12)
                if not ok:
                    return False
    return True


# ----------------------------------------------------------------------------- pins

def test_chunk_slices_are_library_full_attention():
    assert check_slices()


@pytest.mark.parametrize("hq,hk", [(3, 3), (6, 2), (8, 1)])
def test_chunk_slices_gqa_groups(hq, hk):
    assert check_slices(hq=hq, hk=hk)


@pytest.mark.parametrize("name", ["tiny", "video256x2", "streaming"])
def test_chunk_slices_on_workload_prompts(name):
    """The workloads' own prompt layouts, on shrunken chunks (the token counts
    are scaled down, the prompt structure is kept)."""
    cfg = get_config(name)
    lay = cfg.layout
    t = text_layout(cfg)
    qlen = [min(7, lay.q_offsets[c + 1] - lay.q_offsets[c]) for c in range(lay.n_chunks)]
    small = layout_from_chunks([[qlen[c] for c in range(lay.seq_chunks[s], lay.seq_chunks[s + 1])]
                                for s in range(lay.n_seqs)])
    # query-less cache chunks keep no rows; keep the text ranges, shortened
    starts = sorted(set(t.begin) | set(t.end))
    shrink = {x: i * 5 for i, x in enumerate(starts)}
    text = type(t)(tuple(shrink[b] for b in t.begin), tuple(shrink[e] for e in t.end), shrink[t.t_text])
    assert check_slices(lay=small, text=text)


def test_brute_force_loops_tiny_config():
    cfg = get_config("tiny")
    lay, text = cfg.layout, text_layout(cfg)
    inp = make_inputs(lay, 2, 1, 64, "fp32", "ones", 1)
    tx = make_text_inputs(text, 1, 64, "fp32", "uniform", 2)
    rows = np.concatenate([np.arange(0, 5), np.arange(60, 70), np.arange(185, 192)])
    a = (inp["q"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, 0.125)
    o1, l1 = oracle.cross_attention(*a, lay.q_offsets, text, rows=rows)
    sub = inp["q"][rows]
    # the loops take a query stream of the sampled rows: give them a layout of
    # one chunk per row with that row's text range
    offs = tuple(range(len(rows) + 1))
    c_of = oracle.token_chunk_ids(lay.q_offsets, lay.t_q)[rows]
    tsub = type(text)(tuple(text.begin[c] for c in c_of), tuple(text.end[c] for c in c_of), text.t_text)
    o2, l2 = oracle.cross_attention_loops(sub, *a[1:], offs, tsub)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
    assert np.array_equal(np.isinf(l1), np.isinf(l2))
    fin = np.isfinite(l1)
    assert np.allclose(l1[fin], l2[fin], rtol=1e-12, atol=1e-12)


def test_brute_force_loops_mixed():
    lay, text = _mixed_case()
    inp, tx = case(lay, text)
    a = (inp["q"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, 0.6, lay.q_offsets, text)
    o1, l1 = oracle.cross_attention(*a)
    o2, l2 = oracle.cross_attention_loops(*a)
    assert np.allclose(o1, o2, rtol=1e-12, atol=1e-12)
    assert np.array_equal(l1 == -np.inf, l2 == -np.inf)
    assert np.allclose(l1[np.isfinite(l1)], l2[np.isfinite(l2)], rtol=1e-12, atol=1e-12)


def test_text_outside_a_chunk_does_not_leak():
    lay, text = _mixed_case()
    inp, tx = case(lay, text)
    a = lambda k, v: oracle.cross_attention(inp["q"], k, v, tx["q_gain_x"], tx["k_gain_x"], 1e-6, 0.5,  # noqa: E731
                                            lay.q_offsets, text)
    o1, l1 = a(tx["k_x"], tx["v_x"])
    k2, v2 = tx["k_x"].clone(), tx["v_x"].clone()
    k2[6:] = torch.randn(k2[6:].shape, generator=torch.Generator().manual_seed(9))
    v2[6:] = 5.0
    o2, l2 = a(k2, v2)
    for c in range(lay.n_chunks):
        sl = slice(lay.q_offsets[c], lay.q_offsets[c + 1])
        if text.end[c] <= 6:                     # prompt 0 = text [0, 6), or no text
            assert np.array_equal(o1[sl], o2[sl]) and np.array_equal(l1[:, sl], l2[:, sl])
        else:
            assert not np.array_equal(o1[sl], o2[sl])


def test_identical_keys_closed_form():
    assert check_identical_keys()


def test_text_pairs_against_mask():
    for cfg in (get_config("tiny"), get_config("video256x2"), get_config("streaming")):
        t = text_layout(cfg)
        assert oracle.text_pairs(cfg.layout.q_offsets, t) == int(oracle.text_mask(cfg.layout.q_offsets, t).sum())
    lay, text = _mixed_case()
    # by hand: chunks 1, 2 (13 + 7 rows) see 6 keys, chunk 3 (11) and chunk 5 (8) see 19
    assert oracle.text_pairs(lay.q_offsets, text) == (13 + 7) * 6 + (11 + 8) * 19


def test_empty_text_stream():
    lay = streaming_layout(2, 1, 5)
    text = chunk_prompts([None, None, None], [])
    inp = make_inputs(lay, 2, 1, 8, "fp32", "ones", 0)
    tx = make_text_inputs(text, 1, 8, "fp32", "ones", 0)
    o, l = oracle.cross_attention(inp["q"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, 0.3,
                                  lay.q_offsets, text)
    assert o.shape == (5, 2, 8) and np.all(o == 0) and np.all(l == -np.inf)


# ----------------------------------------------------------------------------- planted mistakes

_orig_mask = cross_mod.text_mask
_orig_cross = cross_mod.cross_attention


def _mask_end_inclusive(q_offsets, text, rows=None):
    tq = int(q_offsets[-1])
    qc = dense_mod.token_chunk_ids(q_offsets, tq)
    if rows is not None:
        qc = qc[np.asarray(rows)]
    b = np.asarray(text.begin)[qc][:, None]
    e = np.asarray(text.end)[qc][:, None]
    j = np.arange(int(text.t_text))[None, :]
    return (j >= b) & (j <= e) & (e > b)


def _mask_clean_sees_all(q_offsets, text, rows=None):
    m = _orig_mask(q_offsets, text, rows)
    m[~m.any(axis=1)] = True
    return m


def _v_normalised(q, k, v, qg, kg, eps, scale, q_offsets, text, rows=None, row_block=256):
    v = dense_mod.rms_norm(v, np.ones(dense_mod._as_f64(v).shape[-1]), eps)
    return _orig_cross(q, k, v, qg, kg, eps, scale, q_offsets, text, rows, row_block)


class _QNotNormalised:
    """Stands in for the oracle's `dense` module: rms_norm leaves the query
    tensor (4 heads in check_slices; the text keys have 2) un-normalised, as
    the paper-notes pseudocode's cross branch does."""

    def __getattr__(self, name):
        return getattr(dense_mod, name)

    @staticmethod
    def rms_norm(x, gain, eps):
        x = dense_mod._as_f64(x)
        return x if x.shape[1] == 4 else dense_mod.rms_norm(x, gain, eps)


def _gqa_modulo(q, k, v, qg, kg, eps, scale, q_offsets, text, rows=None, row_block=256):
    hq, hk = q.shape[1], k.shape[1]
    perm = [h % hk for h in range(hq)]
    return _orig_cross(q, dense_mod._as_f64(k)[:, perm], dense_mod._as_f64(v)[:, perm], qg, kg, eps, scale,
                       q_offsets, text, rows, row_block)


@pytest.mark.parametrize("mutant", ["end_inclusive", "clean_sees_all", "v_normalised", "q_not_normalised",
                                    "gqa_modulo"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    """Each mistake planted in the oracle (on the CPU) makes the slice pin fail."""
    if mutant == "end_inclusive":
        monkeypatch.setattr(cross_mod, "text_mask", _mask_end_inclusive)
    elif mutant == "clean_sees_all":
        monkeypatch.setattr(cross_mod, "text_mask", _mask_clean_sees_all)
    elif mutant == "v_normalised":
        monkeypatch.setattr(cross_mod, "cross_attention", _v_normalised)
    elif mutant == "q_not_normalised":
        monkeypatch.setattr(cross_mod, "dense", _QNotNormalised())
    elif mutant == "gqa_modulo":
        monkeypatch.setattr(cross_mod, "cross_attention", _gqa_modulo)
    assert not check_slices(cross_mod.cross_attention, hq=4, hk=2)
