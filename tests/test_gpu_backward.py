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
    # Poison the outputs: every element must be written.
    dq, dk, dv = (torch.full_like(g[n], float("nan")) for n in ("q", "k", "v"))
    grads = plan.backward(g["q"], g["k"], g["v"], out, lse, dout.to(DEV), g["q_gain"], g["k_gain"], eps, sc,
                          dq=dq, dk=dk, dv=dv)
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
    ("last_global", dataclasses.replace(layout_from_chunks([[130, 70], [1, 2, 3], [96, 150], [190, 40]]),
                                        last_global=1)),
    # video 0 is one cached chunk without queries: no row sees its 300 keys (a whole 256-key block among them)
    ("unseen_video", Layout((0, 0, 140, 230), (0, 300, 400, 530), (0, 1, 3))),
]


@pytest.mark.parametrize("name,lay", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("hq,hk", [(6, 2), (8, 1), (3, 3)])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_backward_small(name, lay, hq, hk, d):
    log(f"bf16 backward {name} {hq}/{hk} d={d}")
    errs = check(lay, hq, hk, d, "bf16", seed=hq * 7 + hk + d)
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))


# Layouts with too few dq items to fill the GPU and long tile lists: the
# backward cuts each dq item into pieces of its key-tile list (fp32 partial
# sums, then a merge that finishes the rows). A cached prefix of 8 x 600 keys
# gives lists of 169-188 tiles (2 pieces); 16 x 1100 gives 585 tiles (8
# pieces with 6/2 heads, 7 with 8/1; the planner's fuzz test pins the counts).
# Both end in a ragged query tile; with 8/1 heads an item packs 8 heads of 32
# tokens, with 6/2 one head of 256 tokens.
SPLIT_DQ = [
    ("prefix_8x600", streaming_layout(8, 2, 600)),
    ("prefix_16x1100", streaming_layout(16, 1, 1100)),
]


@pytest.mark.parametrize("name,lay", SPLIT_DQ, ids=[s[0] for s in SPLIT_DQ])
@pytest.mark.parametrize("hq,hk", [(6, 2), (8, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_backward_split_dq_items(name, lay, hq, hk, d):
    log(f"bf16 backward, split dq items: {name} {hq}/{hk} d={d}")
    errs = check(lay, hq, hk, d, "bf16", seed=hq * 11 + hk + d)
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))


FP32_SMALL = SMALL[:4] + SMALL[-2:]


@pytest.mark.parametrize("name,lay", FP32_SMALL, ids=[s[0] for s in FP32_SMALL])
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_backward_small(name, lay, d):
    log(f"fp32 backward {name} d={d}")
    errs = check(lay, 4, 2, d, "fp32", seed=d)
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))


def test_keys_no_row_sees_get_zero_gradients():
    lay = SMALL[-1][1]
    got, ref = run(lay, 6, 2, 128, "bf16", seed=4)
    assert np.all(ref[1][:300] == 0) and np.all(ref[2][:300] == 0)
    assert np.all(got[1][:300] == 0) and np.all(got[2][:300] == 0)


@pytest.mark.parametrize("d", [64, 128])
def test_bf16_backward_scale_and_eps(d):
    lay = layout_from_chunks([[90, 60]])
    check(lay, 4, 2, d, "bf16", seed=3, eps=0.25, scale=0.05)


@pytest.mark.parametrize("lay", [layout_from_chunks([[100, 157, 91]]), streaming_layout(8, 2, 600)],
                         ids=["ragged", "split_dq_items"])
def test_backward_is_deterministic(lay):
    """Two backward calls give bit-identical gradients (no atomics; split
    items' pieces are added in a fixed order)."""
    from block_causal_attention_flash_amd import TrainPlan
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


# ------------------------------------------------------------------ full-size workloads

def _sample_rows(lay, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for c in range(lay.n_chunks):
        a, b = lay.q_offsets[c], lay.q_offsets[c + 1]
        for r in (a, b - 1):
            if a <= r < b:
                rows.add(r)
    rows.update(int(x) for x in rng.integers(0, lay.t_q, n_random))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name,d", [("video480x832", 128), ("video256x2", 128), ("streaming", 128), ("packed8", 128),
                                    ("video480x832", 64)])
def test_backward_full_size(name, d):
    """The workload at full size, in the launch configuration the benchmark
    times: dq of sampled rows (chunk edges and random rows) against the
    oracle; dk and dv of sampled keys of a late chunk (seen by few rows) on
    the smaller workloads; and, over every row and key, properties that hold
    at any size: sum_j dv_jg = sum over g's query rows of dO (softmax rows
    sum to one), <q_i, dq_i> ~ 0 (RMSNorm is scale invariant), all finite.
    480x832 also runs at head_dim 64 (scale 1/8), as `bench.py --head-dim 64
    --backward` times it."""
    import dataclasses
    from workloads import get_config
    from block_causal_attention_flash_amd import TrainPlan
    c = dataclasses.replace(get_config(name), head_dim=d)
    lay = c.layout
    log(f"backward {name} d{d}: generating inputs")
    inp = make_inputs(lay, c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype, c.gain_kind, c.seed)
    dout = torch.from_numpy(np.random.default_rng(c.seed + 7).standard_normal(
        (lay.t_q, c.n_q_heads, c.head_dim), dtype=np.float32)).to(torch.bfloat16)
    g = {n: t.to(DEV) for n, t in inp.items()}
    plan = TrainPlan.from_layout(lay, c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype)
    log(f"backward {name} d{d}: GPU forward + backward")
    out, lse = plan(g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], c.eps, c.scale)
    dq, dk, dv, dgq, dgk = plan.backward(g["q"], g["k"], g["v"], out, lse, dout.to(DEV), g["q_gain"], g["k_gain"],
                                         c.eps, c.scale)
    torch.cuda.synchronize()
    plan.close()
    del out
    for t in (dq, dk, dv, dgq, dgk):
        assert bool(torch.isfinite(t).all())
    # sum of dv over keys, per KV head, against the upstream gradients
    G = c.n_q_heads // c.n_kv_heads
    lhs = dv.double().sum(0)
    rhs = dout.to(DEV).double().reshape(lay.t_q, c.n_kv_heads, G, c.head_dim).sum((0, 2))
    err = float(torch.linalg.vector_norm(lhs - rhs) / torch.linalg.vector_norm(rhs))
    log(f"backward {name} d{d}: sum dv identity rel {err:.2e}")
    assert err <= 1e-2
    # <q, dq> per row, relative to |q| |dq|
    qd = (g["q"].float() * dq.float()).sum(-1).abs()
    ratio = float((qd / (torch.linalg.vector_norm(g["q"].float(), dim=-1)
                         * torch.linalg.vector_norm(dq.float(), dim=-1) + 1e-30)).max())
    log(f"backward {name} d{d}: max |<q, dq>| / (|q| |dq|) {ratio:.2e}")
    assert ratio <= 2e-2
    rows = _sample_rows(lay, 8 if name == "video480x832" else 16, seed=c.seed)
    log(f"backward {name} d{d}: dq oracle on {len(rows)} rows")
    args = (inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], c.eps, c.scale, lay, dout)
    ref = oracle.dq_rows(*args, rows)
    e_dq = rel_l2(dq[torch.as_tensor(rows, device=DEV)].double().cpu().numpy(), ref)
    log(f"backward {name} d{d}: dq rows rel_l2 {e_dq:.2e}")
    assert e_dq <= TOL["bf16"]
    if name in ("video256x2", "streaming"):
        last = lay.n_chunks - 1
        keys = np.random.default_rng(c.seed).integers(lay.kv_offsets[last], lay.kv_offsets[last + 1], 6)
        keys = np.unique(np.concatenate([keys, [lay.kv_offsets[last], lay.kv_offsets[last + 1] - 1]]))
        log(f"backward {name} d{d}: dk/dv oracle on {len(keys)} keys")
        rk, rv = oracle.dkv_keys(*args, keys)
        kk = torch.as_tensor(keys, device=DEV)
        e_dk = rel_l2(dk[kk].double().cpu().numpy(), rk)
        e_dv = rel_l2(dv[kk].double().cpu().numpy(), rv)
        log(f"backward {name} d{d}: dk keys rel_l2 {e_dk:.2e} dv keys rel_l2 {e_dv:.2e}")
        assert e_dk <= TOL["bf16"] and e_dv <= TOL["bf16"]


# ------------------------------------------------------------------ the size limit

def test_kv_stream_at_the_2gib_limit_forward_and_backward():
    """A KV stream 64 KiB under the 2 GiB limit of the bf16 tile images
    (1,048,528 keys x 8 KV heads): a cached prefix of 1,048,428 keys without
    queries, then one chunk of 100 queries with a KV range of 1, so the
    queries see only the last 100 keys. The GPU plans, prepares and addresses
    the whole stream (tile offsets near 2^31); the oracle needs only the last
    chunk, since no query sees the prefix. The prefix's dk and dv must be
    exactly 0 (key blocks no row sees)."""
    from block_causal_attention_flash_amd import TrainPlan
    hq, hk, d, n, prefix = 16, 8, 128, 100, 1_048_428
    lay = Layout((0, 0, n), (0, prefix, prefix + n), (0, 2), kv_range=1)
    sub = Layout((0, n), (0, n), (0, 1))
    small = make_inputs(sub, hq, hk, d, "bf16", "uniform", 21)
    gen = torch.Generator(device=DEV).manual_seed(21)
    k = torch.randn(prefix + n, hk, d, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    v = torch.randn(prefix + n, hk, d, generator=gen, device=DEV, dtype=torch.float32).to(torch.bfloat16)
    k[prefix:] = small["k"].to(DEV)
    v[prefix:] = small["v"].to(DEV)
    q, qg, kg = (small[x].to(DEV) for x in ("q", "q_gain", "k_gain"))
    dout = torch.from_numpy(np.random.default_rng(22).standard_normal((n, hq, d)).astype(np.float32)).to(
        torch.bfloat16)
    sc = 1 / math.sqrt(d)
    log("2 GiB stream: plan, forward, backward")
    plan = TrainPlan.from_layout(lay, hq, hk, d, "bf16")
    out, lse = plan(q, k, v, qg, kg, 1e-6, sc)
    dk, dv = torch.full_like(k, float("nan")), torch.full_like(v, float("nan"))
    dq, dk, dv, dgq, dgk = plan.backward(q, k, v, out, lse, dout.to(DEV), qg, kg, 1e-6, sc, dk=dk, dv=dv)
    torch.cuda.synchronize()
    plan.close()
    assert bool((dk[:prefix] == 0).all()) and bool((dv[:prefix] == 0).all())
    ref_out, ref_lse = oracle.attention(small["q"], small["k"], small["v"], small["q_gain"], small["k_gain"], 1e-6,
                                        sc, sub)
    got_out = out.double().cpu().numpy()
    assert np.max(np.abs(got_out - ref_out)) <= 2e-2 and rel_l2(got_out, ref_out) <= 5e-3
    assert np.max(np.abs(lse.double().cpu().numpy() - ref_lse)) <= 1e-2
    ref = oracle.attention_backward(small["q"], small["k"], small["v"], small["q_gain"], small["k_gain"], 1e-6, sc,
                                    sub, dout)
    got = [dq.double().cpu().numpy(), dk[prefix:].double().cpu().numpy(), dv[prefix:].double().cpu().numpy(),
           dgq.double().cpu().numpy(), dgk.double().cpu().numpy()]
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))
    assert max(errs) <= TOL["bf16"]
