"""GPU parity of the cross-attention's backward (a cross training plan through
magi_attn_bwd, the C ABI) against the fp64 oracle
(oracle.cross_attention_backward and its row/key restrictions).

The GPU backward takes the GPU forward's out and lse, as training does.
Tolerances are the self-attention backward's (relative L2 per gradient):
bf16 1e-2, fp32 1e-5. Rows without text must come back with dq exactly 0,
and text tokens no row sees with dk = dv = 0.
"""
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import (Layout, TextLayout, chunk_prompts, get_config, layout_from_chunks, make_inputs,
                       make_text_inputs, prompt_draw, streaming_layout, text_layout)

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
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def run(lay, text, hq, hk, d, dtype, seed, eps=1e-6, scale=None):
    from block_causal_attention_flash_amd import CrossTrainPlan
    sc = 1.0 / np.sqrt(d) if scale is None else scale
    q = make_inputs(lay, hq, hk, d, dtype, "uniform", seed)["q"]
    tx = make_text_inputs(text, hk, d, dtype, "uniform", seed + 1)
    dout = torch.from_numpy(np.random.default_rng(seed + 7).standard_normal((lay.t_q, hq, d)).astype(np.float32)
                            ).to(q.dtype)
    plan = CrossTrainPlan.from_layout(lay, text, hq, hk, d, dtype)
    g = {n: t.to(DEV) for n, t in tx.items()}
    qd = q.to(DEV)
    # Poison the outputs: every element must be written.
    dq = torch.full_like(qd, float("nan"))
    dk = torch.full_like(g["k_x"], float("nan"))
    dv = torch.full_like(g["v_x"], float("nan"))
    out, lse = plan(qd, g["k_x"], g["v_x"], g["q_gain_x"], g["k_gain_x"], eps, sc)
    grads = plan.backward(qd, g["k_x"], g["v_x"], out, lse, dout.to(DEV), g["q_gain_x"], g["k_gain_x"], eps, sc,
                          dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    got = [t.double().cpu().numpy() for t in grads]
    plan.close()
    ref = oracle.cross_attention_backward(q, tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], eps, sc,
                                          lay.q_offsets, text, dout)
    return got, ref


def check(lay, text, hq, hk, d, dtype, seed, **kw):
    got, ref = run(lay, text, hq, hk, d, dtype, seed, **kw)
    for a in got:
        assert np.all(np.isfinite(a))
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    assert max(errs) <= TOL[dtype], dict(zip(("dq", "dk", "dv", "dq_gain", "dk_gain"), errs))
    # exact zeros on rows without text and on text tokens no row sees (taken
    # from the mask: a one-token prompt also gives the oracle dq = 0 exactly,
    # where dS = P (dP - D) cancels only in exact arithmetic)
    m = oracle.text_mask(lay.q_offsets, text)
    assert np.all(got[0][~m.any(axis=1)] == 0)
    unseen = ~m.any(axis=0)
    assert np.all(got[1][unseen] == 0) and np.all(got[2][unseen] == 0)
    return errs


_PACKED = layout_from_chunks([[64, 64], [1, 2, 3], [200], [33, 95, 7]])
_STREAM = streaming_layout(5, 3, 96)
SMALL = [
    # chunk 0 clean, two ragged prompts
    ("own_prompts", layout_from_chunks([[100, 157, 91]]), chunk_prompts([None, 0, 1], [70, 45])),
    # one prompt per two chunks of each video, first chunk clean; text past the prompts unseen
    ("packed", _PACKED, prompt_draw(_PACKED, 1, 2, seed=11, lo=9, hi=80)),
    # KV cache: cached chunks carry no queries
    ("streaming", _STREAM, prompt_draw(_STREAM, 0, 2, seed=12, lo=20, hi=120)),
    # chunks 0 and 2 share a prompt: two separate runs of rows per text key
    ("two_runs", layout_from_chunks([[130, 70, 96, 150]]), chunk_prompts([0, 1, 0, None], [77, 40])),
    # a prompt longer than 256 keys (several dk/dv items per prompt)
    ("long_prompt", layout_from_chunks([[64, 96]]), chunk_prompts([0, 0], [300])),
]


@pytest.mark.parametrize("name,lay,text", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("hq,hk", [(6, 2), (8, 1), (3, 3)])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_cross_backward_small(name, lay, text, hq, hk, d):
    log(f"bf16 cross backward {name} {hq}/{hk} d={d}")
    errs = check(lay, text, hq, hk, d, "bf16", seed=hq * 7 + hk + d)
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))


@pytest.mark.parametrize("name,lay,text", SMALL, ids=[s[0] for s in SMALL])
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_cross_backward_small(name, lay, text, d):
    log(f"fp32 cross backward {name} d={d}")
    errs = check(lay, text, 4, 2, d, "fp32", seed=d)
    log("  rel_l2 dq {:.2e} dk {:.2e} dv {:.2e} dgq {:.2e} dgk {:.2e}".format(*errs))


@pytest.mark.parametrize("dtype", ["bf16", "fp32"])
def test_cross_backward_without_text(dtype):
    """t_text = 0: every row has out 0; dq and both gain gradients are 0."""
    lay = layout_from_chunks([[40, 72]])
    got, ref = run(lay, TextLayout((0, 0), (0, 0), 0), 4, 2, 128, dtype, seed=3)
    assert got[1].shape == (0, 2, 128) and got[2].shape == (0, 2, 128)
    for a in (got[0], got[3], got[4]):
        assert np.all(a == 0)


def test_cross_backward_is_deterministic():
    from block_causal_attention_flash_amd import CrossTrainPlan
    lay = _PACKED
    text = prompt_draw(lay, 1, 2, seed=5, lo=9, hi=80)
    q = make_inputs(lay, 6, 2, 128, "bf16", "uniform", 5)["q"].to(DEV)
    tx = {n: t.to(DEV) for n, t in make_text_inputs(text, 2, 128, "bf16", "uniform", 6).items()}
    dout = torch.randn(lay.t_q, 6, 128, generator=torch.Generator().manual_seed(1)).to(torch.bfloat16).to(DEV)
    plan = CrossTrainPlan.from_layout(lay, text, 6, 2, 128, "bf16")
    out, lse = plan(q, tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"])
    args = (q, tx["k_x"], tx["v_x"], out, lse, dout, tx["q_gain_x"], tx["k_gain_x"])
    a = [t.cpu() for t in plan.backward(*args)]
    b = [t.cpu() for t in plan.backward(*args)]
    torch.cuda.synchronize()
    plan.close()
    for x, y in zip(a, b):
        assert torch.equal(x, y)


def test_cross_plan_without_training_lists_is_refused():
    from block_causal_attention_flash_amd import CrossPlan, MagiAttnError, magi_attn_bwd
    lay = layout_from_chunks([[64]])
    plan = CrossPlan.from_layout(lay, chunk_prompts([0], [16]), 2, 1, 128, "bf16")
    z = torch.zeros(64, 2, 128, dtype=torch.bfloat16, device=DEV)
    zk = torch.zeros(16, 1, 128, dtype=torch.bfloat16, device=DEV)
    lse = torch.zeros(2, 64, device=DEV)
    with pytest.raises(MagiAttnError) as e:
        magi_attn_bwd(plan.handle, z, zk, zk, z, lse, z)
    assert e.value.status == 1
    plan.close()


# ------------------------------------------------------------------ full-size workloads

@pytest.mark.parametrize("name", ["video480x832", "video256x2", "streaming", "packed8"])
def test_cross_backward_full_size(name):
    """Each workload with its prompts (the benchmark's configuration): dq of
    sampled rows against the oracle (chunk edges, random rows, a row of a
    clean chunk), dk and dv of sampled text keys on the smaller workloads,
    and over every row and key: finite, dq = 0 on rows without text, and
    sum_j dv_jg = sum over g's query rows with text of dO."""
    from block_causal_attention_flash_amd import CrossTrainPlan
    c = get_config(name)
    lay = c.layout
    text = text_layout(c)
    log(f"cross backward {name}: inputs (t_text {text.t_text})")
    q = make_inputs(lay, c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype, c.gain_kind, c.seed)["q"]
    tx = make_text_inputs(text, c.n_kv_heads, c.head_dim, c.dtype, c.gain_kind, c.seed + 100)
    dout = torch.from_numpy(np.random.default_rng(c.seed + 7).standard_normal(
        (lay.t_q, c.n_q_heads, c.head_dim), dtype=np.float32)).to(torch.bfloat16)
    g = {n: t.to(DEV) for n, t in tx.items()}
    qd = q.to(DEV)
    plan = CrossTrainPlan.from_layout(lay, text, c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype)
    log(f"cross backward {name}: GPU forward + backward")
    out, lse = plan(qd, g["k_x"], g["v_x"], g["q_gain_x"], g["k_gain_x"], c.eps, c.scale)
    dq, dk, dv, dgq, dgk = plan.backward(qd, g["k_x"], g["v_x"], out, lse, dout.to(DEV), g["q_gain_x"],
                                         g["k_gain_x"], c.eps, c.scale)
    torch.cuda.synchronize()
    plan.close()
    del out
    for t in (dq, dk, dv, dgq, dgk):
        assert bool(torch.isfinite(t).all())
    qc = np.searchsorted(np.asarray(lay.q_offsets), np.arange(lay.t_q), side="right") - 1
    has_text = (np.asarray(text.end) > np.asarray(text.begin))[qc]
    assert bool((dq[torch.as_tensor(~has_text, device=DEV)] == 0).all())
    G = c.n_q_heads // c.n_kv_heads
    lhs = dv.double().sum(0)
    rhs = dout.to(DEV)[torch.as_tensor(has_text, device=DEV)].double().reshape(-1, c.n_kv_heads, G,
                                                                               c.head_dim).sum((0, 2))
    err = float(torch.linalg.vector_norm(lhs - rhs) / torch.linalg.vector_norm(rhs))
    log(f"cross backward {name}: sum dv identity rel {err:.2e}")
    assert err <= 1e-2
    rng = np.random.default_rng(c.seed)
    rows = set(int(x) for x in rng.choice(np.nonzero(has_text)[0], 8))
    for cc in range(lay.n_chunks):
        a, b = lay.q_offsets[cc], lay.q_offsets[cc + 1]
        if b > a:
            rows.update((a, b - 1))
    rows = np.array(sorted(rows))
    args = (q, tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], c.eps, c.scale, lay.q_offsets, text, dout)
    log(f"cross backward {name}: dq oracle on {len(rows)} rows")
    ref = oracle.cross_dq_rows(*args, rows)
    e_dq = rel_l2(dq[torch.as_tensor(rows, device=DEV)].double().cpu().numpy(), ref)
    log(f"cross backward {name}: dq rows rel_l2 {e_dq:.2e}")
    assert e_dq <= TOL["bf16"]
    if name in ("video256x2", "streaming"):
        keys = np.unique(np.concatenate([rng.integers(0, text.t_text, 6), [0, text.t_text - 1]]))
        log(f"cross backward {name}: dk/dv oracle on {len(keys)} text keys")
        rk, rv = oracle.cross_dkv_keys(*args, keys)
        kk = torch.as_tensor(keys, device=DEV)
        e_dk = rel_l2(dk[kk].double().cpu().numpy(), rk)
        e_dv = rel_l2(dv[kk].double().cpu().numpy(), rv)
        log(f"cross backward {name}: dk keys rel_l2 {e_dk:.2e} dv keys rel_l2 {e_dv:.2e}")
        assert e_dk <= TOL["bf16"] and e_dv <= TOL["bf16"]
