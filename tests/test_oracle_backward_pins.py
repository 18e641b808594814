"""Pins of the fp64 backward oracle (oracle/backward.py) against facts that do
not come from the oracle itself:

  * torch autograd in fp64 through torch's rms_norm, matmul and softmax, with
    the mask built here from the offsets by searchsorted (not by the oracle);
  * central finite differences of L = sum(out * dO) on a tiny case, for every
    coordinate of q, k, v and both gains;
  * exact identities: the value gradients of a KV head sum to the upstream
    gradients of its query rows (softmax rows sum to 1); with eps = 0 the
    RMS-normalised inputs are scale invariant, so <x, dx> = 0 per token and
    head; keys that no row with a gradient sees get exactly zero gradient.
Planted mistakes (a dropped softmax-Jacobian term, a dropped RMSNorm
projection, GQA gradients overwritten instead of summed, a gain gradient of
one head only) each fail a pin. The forward is the MAGI-1 attention of
paperlayer §2 / Figure 1 and §2.2.2, paper-notes §3.2.2 and Figure 15; the
KV range of paperlayer §2.4.4.
"""
import dataclasses

import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import backward as bwd_mod
from workloads import layout_from_chunks, make_inputs, streaming_layout


def mask_from_offsets(lay):
    """Allowed (query, key) pairs, built independently of the oracle."""
    tq, tk = lay.t_q, lay.t_k
    qc = np.searchsorted(np.asarray(lay.q_offsets), np.arange(tq), side="right") - 1
    kc = np.searchsorted(np.asarray(lay.kv_offsets), np.arange(tk), side="right") - 1
    vid = lambda c: np.searchsorted(np.asarray(lay.seq_chunks), c, side="right") - 1  # noqa: E731
    m = (vid(qc)[:, None] == vid(kc)[None, :]) & (kc[None, :] <= qc[:, None])
    if lay.kv_range:
        m &= kc[None, :] > qc[:, None] - lay.kv_range
    if lay.last_global:
        m[vid(qc) == len(lay.seq_chunks) - 2, :] = True
    return torch.from_numpy(m)


def autograd_reference(inp, dout, eps, scale, lay):
    q, k, v = (inp[n].detach().to(torch.float64).requires_grad_(True) for n in ("q", "k", "v"))
    gq = inp["q_gain"].detach().to(torch.float64).requires_grad_(True)
    gk = inp["k_gain"].detach().to(torch.float64).requires_grad_(True)
    d = q.shape[-1]
    group = q.shape[1] // k.shape[1]
    qh = F.rms_norm(q, (d,), gq, eps)
    kh = F.rms_norm(k, (d,), gk, eps).repeat_interleave(group, dim=1)
    vv = v.repeat_interleave(group, dim=1)
    s = scale * torch.matmul(qh.transpose(0, 1), kh.permute(1, 2, 0).contiguous())      # [H, Tq, Tk]
    s = s.masked_fill(~mask_from_offsets(lay)[None], float("-inf"))
    p = torch.softmax(s, dim=-1)
    out = torch.matmul(p, vv.transpose(0, 1).contiguous()).transpose(0, 1)               # [Tq, H, d]
    loss = (out * dout.to(torch.float64)).sum()
    return [t.numpy() for t in torch.autograd.grad(loss, (q, k, v, gq, gk))]


def case(lay, hq, hk, d, seed, gains="uniform"):
    inp = make_inputs(lay, hq, hk, d, "fp32", gains, seed)
    dout = torch.from_numpy(np.random.default_rng(seed + 50).standard_normal((lay.t_q, hq, d)))
    return inp, dout


def oracle_grads(inp, dout, eps, scale, lay):
    return bwd_mod.attention_backward(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], eps, scale, lay,
                                      dout)


LAYOUTS = {
    "packed": layout_from_chunks([[5, 7, 3], [4], [2, 6]]),
    "streaming": streaming_layout(3, 2, 4),
    "window": dataclasses.replace(layout_from_chunks([[3, 4, 2, 5, 3]]), kv_range=2),
    "last_global": dataclasses.replace(layout_from_chunks([[5, 7, 3], [4, 2], [3, 4]]), last_global=1),
}


def check_autograd(lay, hq=4, hk=2, d=8, seed=0, eps=1e-6, scale=0.4):
    inp, dout = case(lay, hq, hk, d, seed)
    got = oracle_grads(inp, dout, eps, scale, lay)
    ref = autograd_reference(inp, dout, eps, scale, lay)
    return all(np.allclose(a, b, rtol=1e-10, atol=1e-11) for a, b in zip(got, ref))


# ----------------------------------------------------------------------------- pins

@pytest.mark.parametrize("name", list(LAYOUTS))
@pytest.mark.parametrize("hq,hk", [(4, 2), (3, 3), (6, 1)])
def test_matches_autograd(name, hq, hk):
    assert check_autograd(LAYOUTS[name], hq, hk)


def test_finite_differences():
    lay = layout_from_chunks([[2, 3], [2]])
    inp, dout = case(lay, 2, 1, 4, seed=3)
    eps, scale = 1e-3, 0.7
    got = oracle_grads(inp, dout, eps, scale, lay)
    names = ("q", "k", "v", "q_gain", "k_gain")
    base = {n: inp[n].to(torch.float64).numpy().copy() for n in names}

    def loss(vals):
        out, _ = oracle.attention(vals["q"], vals["k"], vals["v"], vals["q_gain"], vals["k_gain"], eps, scale, lay)
        return float(np.sum(out * dout.numpy()))

    h = 1e-6
    for gi, n in enumerate(names):
        num = np.zeros_like(base[n])
        for idx in np.ndindex(*base[n].shape):
            plus = {m: base[m].copy() for m in names}
            minus = {m: base[m].copy() for m in names}
            plus[n][idx] += h
            minus[n][idx] -= h
            num[idx] = (loss(plus) - loss(minus)) / (2 * h)
        assert np.allclose(got[gi], num, rtol=1e-6, atol=1e-8), n


def test_value_gradients_sum_to_upstream():
    """sum_j dv_jg = sum over rows i of g's query heads of dO_i, since every
    softmax row sums to one."""
    lay = LAYOUTS["packed"]
    inp, dout = case(lay, 6, 2, 8, seed=4)
    _, _, dv, _, _ = oracle_grads(inp, dout, 1e-6, 0.5, lay)
    do = dout.numpy()
    for g in range(2):
        assert np.allclose(dv[:, g].sum(axis=0), do[:, 3 * g:3 * g + 3].sum(axis=(0, 1)), rtol=1e-12, atol=1e-12)


def test_rms_scale_invariance_without_eps():
    """With eps = 0, q_hat and k_hat do not change when a row of q or k is
    scaled, so the gradient is orthogonal to the row: <x, dx> = 0."""
    lay = LAYOUTS["window"]
    inp, dout = case(lay, 4, 2, 8, seed=5)
    dq, dk, _, _, _ = oracle_grads(inp, dout, 0.0, 0.6, lay)
    q = inp["q"].double().numpy()
    k = inp["k"].double().numpy()
    assert np.max(np.abs(np.sum(q * dq, axis=-1))) < 1e-12
    assert np.max(np.abs(np.sum(k * dk, axis=-1))) < 1e-12
    assert np.max(np.abs(dq)) > 1e-3 and np.max(np.abs(dk)) > 1e-3


def test_unseen_keys_get_no_gradient():
    """Only the first chunk's rows carry a gradient: keys of later chunks
    (and of other videos) get exactly zero dk and dv."""
    lay = LAYOUTS["packed"]
    inp, dout = case(lay, 4, 2, 8, seed=6)
    dout[lay.q_offsets[1]:] = 0
    _, dk, dv, _, _ = oracle_grads(inp, dout, 1e-6, 0.5, lay)
    assert np.all(dk[lay.kv_offsets[1]:] == 0) and np.all(dv[lay.kv_offsets[1]:] == 0)
    assert np.max(np.abs(dk[:lay.kv_offsets[1]])) > 0


@pytest.mark.parametrize("name", list(LAYOUTS))
def test_row_and_key_restrictions_match_the_full_backward(name):
    """dq_rows and dkv_keys (used on samples of full-size layouts) give the
    full backward's rows and keys."""
    lay = LAYOUTS[name]
    inp, dout = case(lay, 6, 2, 8, seed=9)
    args = (inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.5, lay, dout)
    dq, dk, dv, _, _ = bwd_mod.attention_backward(*args)
    rows = np.array([0, 3, lay.t_q - 1])
    keys = np.array([0, lay.t_k // 2, lay.t_k - 1])
    assert np.allclose(bwd_mod.dq_rows(*args, rows), dq[rows], rtol=1e-12, atol=1e-13)
    gk, gv = bwd_mod.dkv_keys(*args, keys)
    assert np.allclose(gk, dk[keys], rtol=1e-12, atol=1e-13)
    assert np.allclose(gv, dv[keys], rtol=1e-12, atol=1e-13)


# ----------------------------------------------------------------------------- planted mistakes

_orig_softmax_backward = bwd_mod.softmax_backward
_orig_rms_backward = bwd_mod.rms_norm_backward
_orig_gain = bwd_mod.gain_gradient
_orig_attention_backward = bwd_mod.attention_backward


def _no_jacobian_term(p, dp):
    return p * dp


def _no_projection(u, r, gain, dxh):
    return gain * dxh / r


def _gain_one_head(u, dxh):
    return np.sum(u[:, :1] * dxh[:, :1], axis=(0, 1))


def _gqa_overwrite(q, k, v, q_gain, k_gain, eps, scale, layout, dout, row_block=256):
    """Mutant: a KV head keeps only the gradient of its last query head."""
    hq, hk = q.shape[1], k.shape[1]
    group = hq // hk
    last = [g * group + group - 1 for g in range(hk)]
    res = _orig_attention_backward(q[:, last], k, v, q_gain, k_gain, eps, scale, layout, dout[:, last], row_block)
    out = list(_orig_attention_backward(q, k, v, q_gain, k_gain, eps, scale, layout, dout, row_block))
    out[1], out[2] = res[1], res[2]
    return tuple(out)


@pytest.mark.parametrize("mutant", ["no_jacobian_term", "no_projection", "gain_one_head", "gqa_overwrite"])
def test_planted_mistakes_are_caught(monkeypatch, mutant):
    if mutant == "no_jacobian_term":
        monkeypatch.setattr(bwd_mod, "softmax_backward", _no_jacobian_term)
    elif mutant == "no_projection":
        monkeypatch.setattr(bwd_mod, "rms_norm_backward", _no_projection)
    elif mutant == "gain_one_head":
        monkeypatch.setattr(bwd_mod, "gain_gradient", _gain_one_head)
    elif mutant == "gqa_overwrite":
        monkeypatch.setattr(bwd_mod, "attention_backward", _gqa_overwrite)
    assert not check_autograd(LAYOUTS["packed"], 4, 2)
