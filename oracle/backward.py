"""fp64 CPU oracle of the backward pass of block-causal QK-RMSNorm GQA attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library.

What is differentiated is the forward of oracle.dense (the MAGI-1 pages:
paperlayer §2 / Figure 1 and §2.2.2, paper-notes §3.2.2 and Figure 15), whose
training needs the gradients of the attention (paperlayer §4.1 and §B.1:
MagiAttention's kernel runs the backward from the forward's saved softmax
statistics). For the upstream gradient dO of out:

  forward    u = x / r,  r = sqrt(mean_d(x^2) + eps),  x_hat = u * g       (q and k)
             s_ij = scale <q_hat_i, k_hat_j> on allowed pairs,  P = softmax_j(s),  O = P V
  backward   dP_ij = <dO_i, v_j>
             dS_ij = P_ij (dP_ij - sum_l P_il dP_il)          (softmax Jacobian)
             dq_hat_i = scale sum_j dS_ij k_hat_j
             dk_hat_j = scale sum_i dS_ij q_hat_i              (over every query head of j's group)
             dv_j     = sum_i P_ij dO_i                        (likewise)
             dx = (g * dx_hat - u * mean_d(u * g * dx_hat)) / r (RMSNorm, per token and head)
             dg = sum over tokens and heads of u * dx_hat      (one gain vector per tensor)

The text cross-attention (oracle.cross: chunk c's rows see the text keys
[begin[c], end[c]) of a separate stream) has the same chain rule over its own
mask; a row without text has out = 0, so its P row is zero and it passes no
gradient. Every function below is that chain rule written out without tiling.
"""
from __future__ import annotations

from typing import Tuple

import numpy as np

from . import cross, dense


def softmax_backward(p: np.ndarray, dp: np.ndarray) -> np.ndarray:
    """dS = P * (dP - rowsum(P * dP)): the Jacobian of a row softmax applied
    to dP. Masked entries have P = 0 and get dS = 0."""
    return p * (dp - np.sum(p * dp, axis=-1, keepdims=True))


def rms_norm_backward(u: np.ndarray, r: np.ndarray, gain: np.ndarray, dxh: np.ndarray) -> np.ndarray:
    """Gradient of x -> x * gain / sqrt(mean(x^2) + eps) with respect to x,
    given u = x / r and the gradient dxh of the output."""
    t = gain * dxh
    return (t - u * np.mean(u * t, axis=-1, keepdims=True)) / r


def gain_gradient(u: np.ndarray, dxh: np.ndarray) -> np.ndarray:
    """Gradient of the shared gain vector: u * dxh summed over tokens and heads."""
    return np.sum(u * dxh, axis=(0, 1))


def _self_mask(layout):
    """Allowed (row, key) pairs of the block-causal self-attention."""
    return lambda rows: dense.block_causal_mask(layout, rows)


def _text_mask(q_offsets, text):
    """Allowed (row, text key) pairs of the cross-attention."""
    return lambda rows: cross.text_mask(q_offsets, text, rows)


def _softmax_rows(s: np.ndarray, mask: np.ndarray) -> np.ndarray:
    """Row softmax over the allowed entries; a row with none is all zero (its
    output is 0 and it passes no gradient)."""
    live = mask.any(axis=1, keepdims=True)
    m = np.max(np.where(mask, s, -np.inf), axis=1, keepdims=True, initial=-np.inf)
    e = np.where(mask, np.exp(s - np.where(live, m, 0.0)), 0.0)
    return e / np.maximum(np.sum(e, axis=1, keepdims=True), np.finfo(np.float64).tiny)


def _backward(q, k, v, q_gain, k_gain, eps, scale, mask_of, dout, row_block):
    q = dense._as_f64(q)
    k = dense._as_f64(k)
    v = dense._as_f64(v)
    do = dense._as_f64(dout)
    gq = dense._as_f64(q_gain)
    gk = dense._as_f64(k_gain)
    tq, hq, d = q.shape
    hk = k.shape[1]
    group = hq // hk
    rq = np.sqrt(np.mean(q * q, axis=-1, keepdims=True) + eps)
    rk = np.sqrt(np.mean(k * k, axis=-1, keepdims=True) + eps)
    uq, uk = q / rq, k / rk
    qh, kh = uq * gq, uk * gk
    dqh = np.zeros_like(q)
    dkh = np.zeros_like(k)
    dv = np.zeros_like(v)
    for r0 in range(0, tq, row_block):
        rows = np.arange(r0, min(tq, r0 + row_block))
        mask = mask_of(rows)
        for h in range(hq):
            g = h // group
            p = _softmax_rows(scale * (qh[rows, h, :] @ kh[:, g, :].T), mask)
            dp = do[rows, h, :] @ v[:, g, :].T
            ds = softmax_backward(p, dp)
            dqh[rows, h, :] = scale * (ds @ kh[:, g, :])
            dkh[:, g, :] += scale * (ds.T @ qh[rows, h, :])
            dv[:, g, :] += p.T @ do[rows, h, :]
    dq = rms_norm_backward(uq, rq, gq, dqh)
    dk = rms_norm_backward(uk, rk, gk, dkh)
    return dq, dk, dv, gain_gradient(uq, dqh), gain_gradient(uk, dkh)


def attention_backward(q, k, v, q_gain, k_gain, eps: float, scale: float, layout, dout, row_block: int = 256
                       ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """Returns dq [T_q,H_q,d], dk, dv [T_k,H_kv,d], dq_gain, dk_gain [d] (fp64)."""
    return _backward(q, k, v, q_gain, k_gain, eps, scale, _self_mask(layout), dout, row_block)


def cross_attention_backward(q, k, v, q_gain, k_gain, eps: float, scale: float, q_offsets, text, dout,
                             row_block: int = 256
                             ) -> Tuple[np.ndarray, np.ndarray, np.ndarray, np.ndarray, np.ndarray]:
    """The cross-attention's gradients: k, v are the text keys/values
    [T_text, H_kv, d] and the gains the cross-attention's own. Returns dq
    [T_q,H_q,d], dk, dv [T_text,H_kv,d], dq_gain, dk_gain [d] (fp64)."""
    return _backward(q, k, v, q_gain, k_gain, eps, scale, _text_mask(q_offsets, text), dout, row_block)


def _row_terms(q, k, v, do, gq, gk, eps, scale, mask_of, rows):
    """For query rows `rows`: q_hat, u, r of the rows, k_hat of all keys,
    and per head the full-row P and dS (the chain rule restricted to rows)."""
    tq, hq, d = q.shape
    hk = k.shape[1]
    group = hq // hk
    rq = np.sqrt(np.mean(q[rows] ** 2, axis=-1, keepdims=True) + eps)
    uq = q[rows] / rq
    rk = np.sqrt(np.mean(k * k, axis=-1, keepdims=True) + eps)
    kh = k / rk * gk
    mask = mask_of(rows)
    ps, dss = [], []
    for h in range(hq):
        g = h // group
        p = _softmax_rows(scale * ((uq[:, h, :] * gq) @ kh[:, g, :].T), mask)
        ps.append(p)
        dss.append(softmax_backward(p, do[rows, h, :] @ v[:, g, :].T))
    return uq, rq, kh, ps, dss


def _dq_rows(q, k, v, q_gain, k_gain, eps, scale, mask_of, dout, rows):
    q, k, v, do = (dense._as_f64(x) for x in (q, k, v, dout))
    gq, gk = dense._as_f64(q_gain), dense._as_f64(k_gain)
    rows = np.asarray(rows, dtype=np.int64)
    hq = q.shape[1]
    group = hq // k.shape[1]
    uq, rq, kh, _, dss = _row_terms(q, k, v, do, gq, gk, eps, scale, mask_of, rows)
    dqh = np.stack([scale * (dss[h] @ kh[:, h // group, :]) for h in range(hq)], axis=1)
    return rms_norm_backward(uq, rq, gq, dqh)


def _dkv_keys(q, k, v, q_gain, k_gain, eps, scale, mask_of, dout, keys):
    q, k, v, do = (dense._as_f64(x) for x in (q, k, v, dout))
    gq, gk = dense._as_f64(q_gain), dense._as_f64(k_gain)
    keys = np.asarray(keys, dtype=np.int64)
    hq, hk = q.shape[1], k.shape[1]
    group = hq // hk
    tq = q.shape[0]
    seen = np.zeros(tq, dtype=bool)
    for r0 in range(0, tq, 1024):
        seen[r0:r0 + 1024] = mask_of(np.arange(r0, min(tq, r0 + 1024)))[:, keys].any(axis=1)
    rows = np.nonzero(seen)[0]
    dkh = np.zeros((len(keys), hk, q.shape[2]))
    dv = np.zeros_like(dkh)
    for b0 in range(0, len(rows), 256):
        rb = rows[b0:b0 + 256]
        uq, _, _, ps, dss = _row_terms(q, k, v, do, gq, gk, eps, scale, mask_of, rb)
        for h in range(hq):
            g = h // group
            dkh[:, g, :] += scale * (dss[h][:, keys].T @ (uq[:, h, :] * gq))
            dv[:, g, :] += ps[h][:, keys].T @ do[rb, h, :]
    rk = np.sqrt(np.mean(k[keys] ** 2, axis=-1, keepdims=True) + eps)
    return rms_norm_backward(k[keys] / rk, rk, gk, dkh), dv


def dq_rows(q, k, v, q_gain, k_gain, eps: float, scale: float, layout, dout, rows) -> np.ndarray:
    """dq of the query rows `rows` only ([R, H_q, d]): the same chain rule as
    attention_backward, evaluated for those rows."""
    return _dq_rows(q, k, v, q_gain, k_gain, eps, scale, _self_mask(layout), dout, rows)


def dkv_keys(q, k, v, q_gain, k_gain, eps: float, scale: float, layout, dout, keys
             ) -> Tuple[np.ndarray, np.ndarray]:
    """dk and dv of the keys `keys` only ([K, H_kv, d] each), summed over
    every query row that sees them (each row's softmax over all its keys)."""
    return _dkv_keys(q, k, v, q_gain, k_gain, eps, scale, _self_mask(layout), dout, keys)


def cross_dq_rows(q, k, v, q_gain, k_gain, eps: float, scale: float, q_offsets, text, dout, rows) -> np.ndarray:
    """dq of the query rows `rows` of the cross-attention ([R, H_q, d])."""
    return _dq_rows(q, k, v, q_gain, k_gain, eps, scale, _text_mask(q_offsets, text), dout, rows)


def cross_dkv_keys(q, k, v, q_gain, k_gain, eps: float, scale: float, q_offsets, text, dout, keys
                   ) -> Tuple[np.ndarray, np.ndarray]:
    """dk and dv of the text keys `keys` of the cross-attention ([K, H_kv, d])."""
    return _dkv_keys(q, k, v, q_gain, k_gain, eps, scale, _text_mask(q_offsets, text), dout, keys)
