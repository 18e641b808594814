"""Pins of the fp64 cross-attention backward oracle
(oracle.cross_attention_backward and its restrictions) against facts that do
not come from the oracle itself:

  * torch autograd in fp64 through torch's rms_norm, matmul and softmax over
    the rows that have text, with the mask built here chunk by chunk (not by
    the oracle); rows without text do not enter the loss (their out is 0);
  * central finite differences of L = sum(out * dO) through the cross forward
    on a tiny case, for every coordinate of q, the text keys and values and
    both gains;
  * exact identities: the value gradients of a KV head sum to the upstream
    gradients of the rows that have text; text keys no row sees, and rows
    without text, get exactly zero gradient.
A planted mistake (the guard of rows without any key dropped, so their
softmax divides 0 by 0) fails a pin. The operation is the cross-attention of
paperlayer §2.2.2 / paper-notes §3.2.2 (QK-Norm and GQA on the text branch),
with chunk-wise prompts (paperlayer §2.2.3) and clean chunks without text
(paper-notes §3.2.6); its training needs these gradients (paperlayer §4.1).
"""
import numpy as np
import pytest
import torch
import torch.nn.functional as F

import oracle
from oracle import backward as bwd_mod
from workloads import TextLayout, chunk_prompts, layout_from_chunks, make_inputs, make_text_inputs


def mask_chunkwise(q_offsets, text):
    """Allowed (row, text key) pairs, filled chunk by chunk."""
    m = np.zeros((q_offsets[-1], text.t_text), dtype=bool)
    for c in range(len(q_offsets) - 1):
        m[q_offsets[c]:q_offsets[c + 1], text.begin[c]:text.end[c]] = True
    return torch.from_numpy(m)


def case(q_chunks, text, hq, hk, d, seed):
    lay = layout_from_chunks([q_chunks])
    inp = make_inputs(lay, hq, hk, d, "fp32", "uniform", seed)
    tx = make_text_inputs(text, hk, d, "fp32", "uniform", seed + 1)
    dout = torch.from_numpy(np.random.default_rng(seed + 50).standard_normal((lay.t_q, hq, d)))
    return lay, inp["q"], tx, dout


def oracle_grads(q, tx, dout, eps, scale, lay, text):
    return oracle.cross_attention_backward(q, tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], eps, scale,
                                           lay.q_offsets, text, dout)


def autograd_reference(q, tx, dout, eps, scale, lay, text):
    q = q.detach().to(torch.float64).requires_grad_(True)
    k, v, gq, gk = (tx[n].detach().to(torch.float64).requires_grad_(True)
                    for n in ("k_x", "v_x", "q_gain_x", "k_gain_x"))
    d = q.shape[-1]
    group = q.shape[1] // k.shape[1]
    mask = mask_chunkwise(lay.q_offsets, text)
    live = mask.any(dim=1)
    qh = F.rms_norm(q, (d,), gq, eps)[live]
    kh = F.rms_norm(k, (d,), gk, eps).repeat_interleave(group, dim=1)
    vv = v.repeat_interleave(group, dim=1)
    s = scale * torch.matmul(qh.transpose(0, 1), kh.permute(1, 2, 0).contiguous())       # [H, live rows, T_text]
    s = s.masked_fill(~mask[live][None], float("-inf"))
    p = torch.softmax(s, dim=-1)
    out = torch.matmul(p, vv.transpose(0, 1).contiguous()).transpose(0, 1)                # [live rows, H, d]
    loss = (out * dout[live].to(torch.float64)).sum()
    return [t.numpy() for t in torch.autograd.grad(loss, (q, k, v, gq, gk))]


# chunk 0 clean; chunks 1, 2 share prompt 0; chunk 3 has prompt 1; chunk 4
# clean; text tokens past the last prompt are seen by no row
TEXTS = {
    "shared_and_clean": ([3, 4, 2, 5, 3], TextLayout((0, 0, 0, 6, 0), (0, 6, 6, 11, 0), 14)),
    "own_prompts": ([5, 7, 3], chunk_prompts([0, 1, 2], [4, 1, 6])),
    "two_runs": ([3, 4, 2, 5], TextLayout((0, 5, 0, 1), (5, 9, 5, 4), 9)),     # chunks 0 and 2 share, 3 overlaps
}


@pytest.mark.parametrize("name", list(TEXTS))
@pytest.mark.parametrize("hq,hk", [(4, 2), (3, 3), (6, 1)])
def test_matches_autograd(name, hq, hk):
    chunks, text = TEXTS[name]
    lay, q, tx, dout = case(chunks, text, hq, hk, 8, seed=hq + 3 * hk)
    got = oracle_grads(q, tx, dout, 1e-6, 0.4, lay, text)
    ref = autograd_reference(q, tx, dout, 1e-6, 0.4, lay, text)
    for a, b in zip(got, ref):
        assert np.allclose(a, b, rtol=1e-10, atol=1e-11)


def test_finite_differences():
    text = TextLayout((0, 0, 1), (0, 3, 4), 5)          # chunk 0 clean, text token 4 unseen
    lay, q, tx, dout = case([2, 2, 1], text, 2, 1, 4, seed=7)
    eps, scale = 1e-3, 0.7
    got = oracle_grads(q, tx, dout, eps, scale, lay, text)
    base = {"q": q.to(torch.float64).numpy().copy()}
    base.update({n: tx[n].to(torch.float64).numpy().copy() for n in ("k_x", "v_x", "q_gain_x", "k_gain_x")})
    names = ("q", "k_x", "v_x", "q_gain_x", "k_gain_x")

    def loss(vals):
        out, _ = oracle.cross_attention(vals["q"], vals["k_x"], vals["v_x"], vals["q_gain_x"], vals["k_gain_x"],
                                        eps, scale, lay.q_offsets, text)
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


def test_value_gradients_sum_to_the_upstream_of_rows_with_text():
    chunks, text = TEXTS["shared_and_clean"]
    lay, q, tx, dout = case(chunks, text, 6, 2, 8, seed=4)
    _, _, dv, _, _ = oracle_grads(q, tx, dout, 1e-6, 0.5, lay, text)
    live = mask_chunkwise(lay.q_offsets, text).any(dim=1).numpy()
    do = dout.numpy()
    for g in range(2):
        assert np.allclose(dv[:, g].sum(axis=0), do[live][:, 3 * g:3 * g + 3].sum(axis=(0, 1)), rtol=1e-12,
                           atol=1e-12)


def test_rows_without_text_and_unseen_keys_get_no_gradient():
    chunks, text = TEXTS["shared_and_clean"]
    lay, q, tx, dout = case(chunks, text, 4, 2, 8, seed=6)
    dq, dk, dv, _, _ = oracle_grads(q, tx, dout, 1e-6, 0.5, lay, text)
    live = mask_chunkwise(lay.q_offsets, text).any(dim=1).numpy()
    assert np.all(dq[~live] == 0) and np.max(np.abs(dq[live])) > 0
    assert np.all(dk[11:] == 0) and np.all(dv[11:] == 0)
    assert np.max(np.abs(dk[:11])) > 0


def test_no_text_at_all():
    text = TextLayout((0, 0), (0, 0), 0)
    lay, q, tx, dout = case([3, 2], text, 2, 1, 4, seed=8)
    dq, dk, dv, dgq, dgk = oracle_grads(q, tx, dout, 1e-6, 0.5, lay, text)
    assert dk.shape == (0, 1, 4) and dv.shape == (0, 1, 4)
    assert np.all(dq == 0) and np.all(dgq == 0) and np.all(dgk == 0)


@pytest.mark.parametrize("name", list(TEXTS))
def test_row_and_key_restrictions_match_the_full_backward(name):
    chunks, text = TEXTS[name]
    lay, q, tx, dout = case(chunks, text, 6, 2, 8, seed=9)
    args = (q, tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, 0.5, lay.q_offsets, text, dout)
    dq, dk, dv, _, _ = oracle.cross_attention_backward(*args)
    rows = np.array([0, 3, lay.t_q - 1])
    keys = np.array([0, text.t_text // 2, text.t_text - 1])
    assert np.allclose(oracle.cross_dq_rows(*args, rows), dq[rows], rtol=1e-12, atol=1e-13)
    gk, gv = oracle.cross_dkv_keys(*args, keys)
    assert np.allclose(gk, dk[keys], rtol=1e-12, atol=1e-13)
    assert np.allclose(gv, dv[keys], rtol=1e-12, atol=1e-13)


def _unguarded_softmax(s, mask):
    e = np.where(mask, np.exp(s - np.max(np.where(mask, s, -np.inf), axis=1, keepdims=True)), 0.0)
    return e / np.sum(e, axis=1, keepdims=True)


def test_planted_empty_row_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(bwd_mod, "_softmax_rows", _unguarded_softmax)
    chunks, text = TEXTS["shared_and_clean"]
    lay, q, tx, dout = case(chunks, text, 4, 2, 8, seed=1)
    with np.errstate(invalid="ignore", divide="ignore"):
        got = oracle_grads(q, tx, dout, 1e-6, 0.4, lay, text)
    ref = autograd_reference(q, tx, dout, 1e-6, 0.4, lay, text)
    assert not all(np.allclose(a, b, rtol=1e-10, atol=1e-11) for a, b in zip(got, ref))
