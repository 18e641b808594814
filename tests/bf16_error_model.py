"""First-order error model of bf16 attention, used to derive tolerances.

A bf16 implementation of the attention in the MAGI-1 pages (paperlayer §2.2.2,
paper-notes §3.2.2: QK-normalised, block-causal softmax attention) rounds the
two normalised operands of the Q K^T product to bf16 once each, rounds P to
bf16 for the P V product and rounds the output. Round-to-nearest-even has a
relative error of at most 2^-8; over values spread across a binade its RMS is
taken as RHO = 2^-8 / sqrt(3) (the RMS of a uniform error on [-2^-8, 2^-8]).

Propagated to first order:
  * logit s_ij = scale <q_hat_i, k_hat_j> (nats): both operands' roundings give
    an error of RMS sigma_ij = sqrt(2) RHO scale sqrt(sum_c q_hat_ic^2 k_hat_jc^2)
    (independent of how the per-channel gains are split between the operands);
  * output: d out_i = sum_j p_ij ds_ij (v_j - out_i) + (P rounding) + (output
    rounding); with independent errors its RMS per element is
      e_id^2 = sum_j p_ij^2 sigma_ij^2 (v_jd - out_id)^2 + RHO^2 sum_j p_ij^2 v_jd^2
               + RHO^2 out_id^2;
  * log-sum-exp: d lse_i = sum_j p_ij ds_ij, whose RMS is at most
    sigma_i = sqrt(sum_j p_ij sigma_ij^2) (the query operand's rounding is shared
    by all keys of the row, and Jensen's inequality bounds its part by the same
    p-weighted mean).

The tolerances take the fixed values (out max-abs 2e-2, rel-L2 5e-3; lse 1e-2) or these first-order estimates,
whichever is larger:
  max-abs of out <= max(2e-2, Z_OUT e_id) per element;
  rel-L2 of out  <= max(5e-3, ||e|| / ||out||);
  lse            <= max(1e-2, Z_LSE sigma_i) per row.
The factors are pinned on the CPU (tests/test_error_model_pins.py) against the
oracle evaluated on bf16-rounded operands; with unit gains the fixed values
bind, and they stop binding as the gains (hence the logits) grow, since bf16
rounding is relative.

Test infrastructure only: it reuses the oracle's normalisation and mask and
runs on the CPU in float64.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence

import numpy as np

import oracle

RHO = 2.0 ** -8 / math.sqrt(3.0)
Z_OUT = 6.0
Z_LSE = 5.0
FIXED_MAXABS, FIXED_RL2, FIXED_LSE = 2e-2, 5e-3, 1e-2


def _f64(x):
    if hasattr(x, "detach"):
        import torch
        return x.detach().cpu().to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def predicted_errors(q, k, v, q_gain, k_gain, eps: float, scale: float, layout,
                     rows: Optional[Sequence[int]] = None, row_block: int = 256):
    """Returns (out, lse, e_out, sigma_lse): the exact (fp64) attention of
    `rows` (default all), the first-order RMS error of each output element and
    the RMS bound of each row's log-sum-exp error (nats), shapes [R, H_q, d],
    [H_q, R], [R, H_q, d], [H_q, R]."""
    q, k, v = _f64(q), _f64(k), _f64(v)
    tq, hq, d = q.shape
    hk = k.shape[1]
    group = hq // hk
    rows = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    qh = oracle.rms_norm(q[rows], q_gain, eps)
    kh = oracle.rms_norm(k, k_gain, eps)
    kh2 = kh * kh
    out = np.zeros((len(rows), hq, d))
    lse = np.zeros((hq, len(rows)))
    e = np.zeros((len(rows), hq, d))
    sig = np.zeros((hq, len(rows)))
    c2 = 2.0 * (RHO * scale) ** 2
    for r0 in range(0, len(rows), row_block):
        sel = slice(r0, min(len(rows), r0 + row_block))
        mask = oracle.block_causal_mask(layout, rows[sel])
        for h in range(hq):
            g = h // group
            s = scale * (qh[sel, h] @ kh[:, g].T)
            s = np.where(mask, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            p = np.exp(s - m)
            l = np.sum(p, axis=1, keepdims=True)
            p /= l
            vg = v[:, g]
            o = p @ vg
            out[sel, h] = o
            lse[h, sel] = (m + np.log(l))[:, 0]
            s2 = c2 * ((qh[sel, h] ** 2) @ kh2[:, g].T)          # sigma_ij^2
            w = p * p * s2
            var_logit = w @ (vg * vg) - 2.0 * o * (w @ vg) + o * o * np.sum(w, axis=1, keepdims=True)
            var_p = RHO ** 2 * ((p * p) @ (vg * vg))
            e[sel, h] = np.sqrt(np.maximum(var_logit, 0.0) + var_p + (RHO * o) ** 2)
            sig[h, sel] = np.sqrt(np.sum(p * s2, axis=1))
    return out, lse, e, sig


def check(got_out, got_lse, ref_out, ref_lse, e_out, sigma_lse, few_key_rows=None):
    """Asserts the tolerances above; returns (rel_l2, max_abs, lse_err, ratios)
    where ratios are each error over its tolerance. `few_key_rows` ([H_q, R]
    bool, optional) restricts the derived LSE bound to rows that see few keys;
    the other rows keep the fixed 1e-2."""
    got_out = np.asarray(got_out, dtype=np.float64)
    got_lse = np.asarray(got_lse, dtype=np.float64)
    assert np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_lse))
    diff = np.abs(got_out - ref_out)
    tol_el = np.maximum(FIXED_MAXABS, Z_OUT * e_out)
    rl2 = float(np.linalg.norm(got_out - ref_out) / np.linalg.norm(ref_out))
    tol_rl2 = max(FIXED_RL2, float(np.linalg.norm(e_out) / np.linalg.norm(ref_out)))
    lse_err = np.abs(got_lse - ref_lse)
    tol_lse = np.maximum(FIXED_LSE, Z_LSE * sigma_lse)
    if few_key_rows is not None:
        tol_lse = np.where(few_key_rows, tol_lse, FIXED_LSE)
    ratios = (float(np.max(diff / tol_el)), rl2 / tol_rl2, float(np.max(lse_err / tol_lse)))
    assert ratios[0] <= 1.0 and ratios[1] <= 1.0 and ratios[2] <= 1.0, (ratios, float(diff.max()), rl2,
                                                                        float(lse_err.max()))
    return rl2, float(diff.max()), float(lse_err.max()), ratios


def lse_tolerance(q, k, q_gain, k_gain, eps: float, scale: float, mask, few_keys: int = 8):
    """[H_q, T_q] LSE tolerance for a dense mask [T_q, T_k]: the fixed 1e-2
    for rows that see at least `few_keys` keys; for rows with fewer (whose LSE
    is close to one logit, with nothing averaged out) max(1e-2, Z_LSE * s_i),
    s_i = sqrt(2) RHO scale sqrt(max_j sum_c q_hat_ic^2 k_hat_jc^2) over the
    row's keys, the largest RMS logit error among them. Rows without keys get
    0 (their LSE is -inf on both sides and compared separately)."""
    q, k = _f64(q), _f64(k)
    hq, hk = q.shape[1], k.shape[1]
    qh2 = oracle.rms_norm(q, q_gain, eps) ** 2
    kh2 = oracle.rms_norm(k, k_gain, eps) ** 2
    mask = np.asarray(mask, dtype=bool)
    n_keys = mask.sum(axis=1)
    tol = np.zeros((hq, q.shape[0]))
    for h in range(hq):
        s2 = np.where(mask, qh2[:, h] @ kh2[:, h // (hq // hk)].T, 0.0)
        sig = math.sqrt(2.0) * RHO * scale * np.sqrt(s2.max(axis=1))
        few = np.maximum(FIXED_LSE, Z_LSE * sig)
        tol[h] = np.where(n_keys >= few_keys, FIXED_LSE, np.where(n_keys > 0, few, 0.0))
    return tol
