"""CPU pins of the bf16 error model that the large-gain GPU tests take their
tolerances from (tests/bf16_error_model.py).

The model is checked against the oracle's own arithmetic applied to operands
rounded to bf16 the way any bf16 implementation must: the two normalised
operands of Q K^T once each (all per-channel gains on the query side, the
temperature outside), P before the P V product, and the output; the row sum is
taken before P's rounding. Nothing here runs the HIP library.
"""
import math

import numpy as np
import pytest
import torch

import oracle
from bf16_error_model import FIXED_LSE, FIXED_MAXABS, check, predicted_errors
from workloads import Layout, layout_from_chunks, make_inputs


def bf16(x):
    return torch.from_numpy(np.ascontiguousarray(x, dtype=np.float64)).to(torch.bfloat16).to(torch.float64).numpy()


def rounded_operand_attention(inp, hq, hk, eps, scale, layout):
    """Masked softmax attention (fp64) from bf16-rounded operands:
    a = bf16(q / rms(q) * g_q * g_k), b = bf16(k / rms(k)), s = scale <a, b>,
    P rounded to bf16 for the product, the sum of the unrounded P, the output
    rounded to bf16."""
    q = inp["q"].double().numpy()
    k = inp["k"].double().numpy()
    v = inp["v"].double().numpy()
    g = inp["q_gain"].double().numpy() * inp["k_gain"].double().numpy()
    a = bf16(q / np.sqrt(np.mean(q * q, -1, keepdims=True) + eps) * g)
    b = bf16(k / np.sqrt(np.mean(k * k, -1, keepdims=True) + eps))
    mask = oracle.block_causal_mask(layout)
    out = np.zeros(q.shape)
    lse = np.zeros((hq, q.shape[0]))
    for h in range(hq):
        kv = h // (hq // hk)
        s = np.where(mask, scale * (a[:, h] @ b[:, kv].T), -np.inf)
        m = s.max(1, keepdims=True)
        e = np.exp(s - m)
        l = e.sum(1, keepdims=True)
        out[:, h] = bf16((bf16(e) @ v[:, kv]) / l)
        lse[h] = (m + np.log(l))[:, 0]
    return out, lse


LAYOUTS = [
    ("three_chunks_ragged", layout_from_chunks([[100, 157, 91]])),
    ("packed_videos", layout_from_chunks([[64, 64], [1, 2, 3], [200], [33, 95, 7]])),
    ("kv_cache_mixed", Layout((0, 0, 0, 77, 150, 150, 260), (0, 64, 130, 200, 333, 400, 470), (0, 4, 6))),
]


@pytest.mark.parametrize("gain_product", [1.0, 2.25, 4.0, 9.0])
@pytest.mark.parametrize("name,layout", LAYOUTS, ids=[n for n, _ in LAYOUTS])
def test_model_covers_bf16_operand_rounding(name, layout, gain_product):
    """Errors of the rounded-operand attention stay within the derived
    tolerances for uniform gain products from 1 to 9 (logits up to 9x those
    of unit gains), in two head layouts and two seeds each."""
    sc = 1.0 / math.sqrt(128)
    worst = [0.0, 0.0, 0.0]
    for hq, hk in ((6, 2), (8, 1)):
        for seed in (5, 6):
            inp = make_inputs(layout, hq, hk, 128, "bf16", "ones", seed)
            inp["q_gain"] = inp["q_gain"] * math.sqrt(gain_product)
            inp["k_gain"] = inp["k_gain"] * math.sqrt(gain_product)
            ref_out, ref_lse, e, sig = predicted_errors(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"],
                                                        1e-6, sc, layout)
            got_out, got_lse = rounded_operand_attention(inp, hq, hk, 1e-6, sc, layout)
            _, _, _, ratios = check(got_out, got_lse, ref_out, ref_lse, e, sig)
            worst = [max(a, b) for a, b in zip(worst, ratios)]
    print(f"{name} G={gain_product}: error / tolerance: max-abs {worst[0]:.2f} rel-L2 {worst[1]:.2f} lse {worst[2]:.2f}")


def test_model_reproduces_the_oracle():
    """predicted_errors returns the oracle's own out and lse."""
    lay = LAYOUTS[0][1]
    inp = make_inputs(lay, 6, 2, 128, "bf16", "uniform", 3)
    sc = 1.0 / math.sqrt(128)
    out, lse, _, _ = predicted_errors(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    assert np.max(np.abs(out - ro)) < 1e-12 and np.max(np.abs(lse - rl)) < 1e-12


def test_model_is_not_vacuous():
    """At gain product 4 the rounded-operand errors exceed the fixed 2e-2 /
    1e-2 somewhere (so the derived bounds are needed), and the rel-L2 bound is
    within a factor 1.5 of the error it covers; with unit gains the fixed
    tolerances bind everywhere. A planted output error of 0.05 or an LSE shift
    of 0.03 fails the tolerances at unit gains."""
    lay = LAYOUTS[2][1]
    sc = 1.0 / math.sqrt(128)
    inp = make_inputs(lay, 8, 1, 128, "bf16", "ones", 5)
    inp4 = dict(inp, q_gain=inp["q_gain"] * 2.0, k_gain=inp["k_gain"] * 2.0)
    ro, rl, e, sig = predicted_errors(inp4["q"], inp4["k"], inp4["v"], inp4["q_gain"], inp4["k_gain"], 1e-6, sc, lay)
    go, gl = rounded_operand_attention(inp4, 8, 1, 1e-6, sc, lay)
    assert np.max(np.abs(go - ro)) > FIXED_MAXABS or np.max(np.abs(gl - rl)) > FIXED_LSE
    rl2, _, _, ratios = check(go, gl, ro, rl, e, sig)
    assert ratios[1] > 1 / 1.5, ratios

    ro, rl, e, sig = predicted_errors(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    assert np.all(6.0 * e < FIXED_MAXABS) and np.linalg.norm(e) / np.linalg.norm(ro) < 5e-3
    go, gl = rounded_operand_attention(inp, 8, 1, 1e-6, sc, lay)
    check(go, gl, ro, rl, e, sig)
    bad = go.copy()
    bad[100, 3, 7] += 0.05
    with pytest.raises(AssertionError):
        check(bad, gl, ro, rl, e, sig)
    badl = gl.copy()
    badl[3, 250] += 0.03
    with pytest.raises(AssertionError):
        check(go, badl, ro, rl, e, sig)
