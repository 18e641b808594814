"""GPU parity of the backward (magi_attn_bwd, through the C ABI) against the
fp64 oracle (oracle.attention_backward).

The GPU backward takes the GPU forward's out and lse, as training does; the
oracle differentiates the exact forward. Tolerances (relative L2 per
gradient; the gain gradients are sums over all rows):
  bf16: dq, dk, dv <= 1e-2 (the forward's bf16 operand rounding, now on five
        products, with P and dS rounded to bf16 as matrix operands and
        dS = P (dP - D) a difference), gain gradients <= 1e-2;
  fp32: every gradient <= 1e-5.
"""
import dataclasses
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import Layout, layout_from_chunks, make_inputs, streaming_layout

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
TOL = {"bf16": 1e-2, "fp32": 1e-5}


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_attention_flash_amd  # noqa: F401
    return built_lib


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def rel_l2(got, ref):
    return float(np.linalg.norm(got - ref) / max(np.linalg.norm(ref), 1e-300))


def run(lay, hq, hk, d, dtype, seed, eps=1e-6, scale=None):
    from block_causal_attention_flash_amd import TrainPlan
    sc = 1.0 / math.sqrt(d) if scale is None else scale
    inp = make_inputs(lay, hq, hk, d, dtype, "uniform", seed)
    tdt = inp["q"].dtype
    dout = torch.from_numpy(np.random.default_rng(seed + 7).standard_normal((lay.t_q, hq, d)).astype(np.float32)).to(tdt)
    plan = TrainPlan.from_layout(lay, hq, hk, d, dtype)
    g = {n: t.to(DEV) for n, t in inp.items()}
    out, lse = plan(g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], eps, sc)
    grads = plan.backward(g["q"], g["k"], g["v"], out, lse, dout.to(DEV), g["q_gain"], g["k_gain"], eps, sc)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in grads]
    plan.close()
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], eps, sc, lay, dout)
    return got, ref


def check(lay, hq, hk, d, dtype, seed, **kw):
    got, ref = run(lay, hq, hk, d, dtype, seed, **kw)
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    for a in got:
        assert np.all(np.isfinite(a))
    assert max(errs) <= TOL[dtype], dict(zip(("dq", "dk", "dv", "dq_gain", "dk_gain"), errs))
    return errs


SMALL = [
    ("one_chunk_ragged", layout_from_chunks([[300]])),
    ("three_chunks_ragged", layout_from_chunks([[100, 157, 91]])),
    ("packed_videos", layout_from_chunks([[64, 64], [1, 2, 3], [200], [33, 95, 7]])),
    ("streaming", streaming_layout(5, 3, 96)),
    ("kv_cache_mixed", Layout((0, 0, 0, 77, 150, 150, 260), (0, 64, 130, 200, 333, 400, 470), (0, 4, 6))),
    ("window", dataclasses.replace(layout_from_chunks([[130, 70, 96, 150], [190, 40]]), kv_range=2)),
]


@pytest.mark.parametrize("name,lay", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("hq,hk", [(6, 2), (8, 1), (3, 3)])
def test_bf16_backward_small(name, lay, hq, hk):
    log(f"bf16 backward {name} {hq}/{hk}")
    errs = check(lay, hq, hk, 128, "bf16", seed=hq * 7 + hk)
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))


@pytest.mark.parametrize("name,lay", SMALL[:4], ids=[s[0] for s in SMALL[:4]])
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_backward_small(name, lay, d):
    log(f"fp32 backward {name} d={d}")
    errs = check(lay, 4, 2, d, "fp32", seed=d)
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))


def test_bf16_backward_scale_and_eps():
    lay = layout_from_chunks([[90, 60]])
    check(lay, 4, 2, 128, "bf16", seed=3, eps=0.25, scale=0.05)


def test_backward_is_deterministic():
    """Two backward calls give bit-identical gradients (no atomics)."""
    from block_causal_attention_flash_amd import TrainPlan
    lay = layout_from_chunks([[100, 157, 91]])
    inp = make_inputs(lay, 6, 2, 128, "bf16", "uniform", 5)
    g = {n: t.to(DEV) for n, t in inp.items()}
    dout = torch.randn(lay.t_q, 6, 128, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(DEV)
    plan = TrainPlan.from_layout(lay, 6, 2, 128, "bf16")
    out, lse = plan(g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"])
    a = [t.cpu() for t in plan.backward(g["q"], g["k"], g["v"], out, lse, dout, g["q_gain"], g["k_gain"])]
    b = [t.cpu() for t in plan.backward(g["q"], g["k"], g["v"], out, lse, dout, g["q_gain"], g["k_gain"])]
    torch.cuda.synchronize()
    plan.close()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_backward_needs_a_training_plan():
    from block_causal_attention_flash_amd import MagiAttnError, Plan, magi_attn_bwd
    lay = layout_from_chunks([[64]])
    plan = Plan.from_layout(lay, 2, 1, 128, "bf16")
    z = torch.zeros(64, 2, 128, dtype=torch.bfloat16, device=DEV)
    zk = torch.zeros(64, 1, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(2, 64, device=DEV)
    with pytest.raises(MagiAttnError) as e:
        magi_attn_bwd(plan.handle, z, zk, zk, z, lse, z)
    assert e.value.status == 1
    plan.close()
