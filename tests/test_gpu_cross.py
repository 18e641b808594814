"""GPU parity of the text cross-attention and of the parallel (self + cross)
launch, through the C ABI, against the fp64 CPU oracles (oracle.attention,
oracle.cross_attention).

Tolerances as for the self-attention: bf16 -- max-abs <= 2e-2, relative L2
<= 5e-3 on the output; fp32 -- relative L2 <= 1e-5, LSE <= 1e-5. The bf16
LSE is held to max(1e-2, B) per row, B the first-order bound of the logit
rounding error (lse_bound): a prompt of a few tokens averages nothing out,
and with one key the LSE is that key's logit. Rows that see no text (chunks
without a prompt) must be exactly 0 with lse = -inf on both sides.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import (CONFIGS, Layout, chunk_prompts, get_config, layout_from_chunks, make_inputs,
                       make_text_inputs, streaming_layout, text_layout)

pytestmark = pytest.mark.gpu

BF16_MAXABS, BF16_RL2, BF16_LSE = 2e-2, 5e-3, 1e-2
FP32_RL2, FP32_LSE = 1e-5, 1e-5
DEV = "cuda:0"


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_attention_flash_amd  # noqa: F401
    return built_lib


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def lse_bound(q, q_gain, k_gain, scale, eps=1e-6, rows=None):
    """[H, R] first-order bound on the bf16 path's LSE error. The kernel
    rounds the folded query q' = rms(q) * g_q * g_k * scale and the normalised
    key k_hat to bf16 (unit roundoff 2^-8 each) and accumulates in fp32, so
    |d lse| <= max_j |d s_ij| <= 2^-7 sum_d |q'_d k_hat_jd| <= 2^-7 |q'| |k_hat_j|
    with |k_hat_j| <= sqrt(d) (unit RMS)."""
    q = q.double() if rows is None else q.double()[torch.as_tensor(rows)]
    d = q.shape[-1]
    qn = q / torch.sqrt((q * q).mean(-1, keepdim=True) + eps) * (q_gain.double() * k_gain.double() * scale)
    return (2.0 ** -7 * math.sqrt(d) * torch.linalg.vector_norm(qn, dim=-1)).T.numpy()


def compare(got_out, got_lse, ref_out, ref_lse, dtype, lse_tol=None):
    """Element-wise parity; rows where the oracle has lse = -inf (no key)
    must be exactly zero with lse = -inf on the GPU too. lse_tol: optional
    [H, R] per-row LSE bound (bf16), used where it exceeds 1e-2."""
    dead = np.isneginf(ref_lse)                                  # [H, R]
    assert np.array_equal(np.isneginf(got_lse), dead)
    dead_rows = dead.T[..., None]                                # [R, H, 1]
    assert np.all(np.where(dead_rows, got_out, 0.0) == 0.0)
    live = ~dead
    assert np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_lse[live]))
    if not live.any():
        return 0.0, 0.0, 0.0
    diff = got_out - ref_out
    rl2 = float(np.linalg.norm(diff) / np.linalg.norm(ref_out))
    mabs = float(np.max(np.abs(diff)))
    lerr = float(np.max(np.abs(got_lse[live] - ref_lse[live])))
    if dtype == "bf16":
        tol = BF16_LSE if lse_tol is None else np.maximum(BF16_LSE, lse_tol)[live]
        assert np.all(np.abs(got_lse[live] - ref_lse[live]) <= tol), lerr
        assert mabs <= BF16_MAXABS and rl2 <= BF16_RL2, (mabs, rl2, lerr)
    else:
        assert rl2 <= FP32_RL2 and lerr <= FP32_LSE, (rl2, lerr)
    return rl2, mabs, lerr


def np64(t):
    return t.double().cpu().numpy()


def inputs(lay, text, hq, hk, d, dtype, seed, distinct_qx=False):
    inp = make_inputs(lay, hq, hk, d, dtype, "uniform", seed)
    tx = make_text_inputs(text, hk, d, dtype, "uniform", seed + 1)
    tx["q_x"] = make_inputs(lay, hq, hk, d, dtype, "ones", seed + 2)["q"] if distinct_qx else inp["q"]
    return inp, tx


def run_cross(lay, text, tx, q, hq, hk, d, dtype, scale):
    from block_causal_attention_flash_amd import CrossPlan
    plan = CrossPlan.from_layout(lay, text, hq, hk, d, dtype)
    out, lse = plan(q.to(DEV), tx["k_x"].to(DEV), tx["v_x"].to(DEV), tx["q_gain_x"].to(DEV),
                    tx["k_gain_x"].to(DEV), 1e-6, scale)
    torch.cuda.synchronize()
    res = np64(out), np64(lse)
    plan.close()
    return res


def run_parallel(lay, text, inp, tx, hq, hk, d, dtype, scale, scale_x, same_q=False):
    from block_causal_attention_flash_amd import ParallelPlan
    plan = ParallelPlan.from_layout(lay, text, hq, hk, d, dtype)
    g = lambda t: t.to(DEV)  # noqa: E731
    out, lse, out_x, lse_x = plan(g(inp["q"]), g(inp["k"]), g(inp["v"]), g(tx["k_x"]), g(tx["v_x"]),
                                  q_x=None if same_q else g(tx["q_x"]), q_gain=g(inp["q_gain"]),
                                  k_gain=g(inp["k_gain"]), q_gain_x=g(tx["q_gain_x"]), k_gain_x=g(tx["k_gain_x"]),
                                  rms_eps=1e-6, scale=scale, scale_x=scale_x)
    torch.cuda.synchronize()
    res = np64(out), np64(lse), np64(out_x), np64(lse_x)
    plan.close()
    return res


def ref_cross(lay, text, tx, scale, rows=None):
    return oracle.cross_attention(tx["q_x"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, scale,
                                  lay.q_offsets, text, rows=rows)


def tol_cross(tx, scale, rows=None):
    return lse_bound(tx["q_x"], tx["q_gain_x"], tx["k_gain_x"], scale, rows=rows)


# ------------------------------------------------------------------ small layouts

def _cases():
    """Layouts with chunk-wise prompts: clean chunks, prompts shared by
    several chunks and by two videos, prompt lengths off the 32-key tile
    grid, query tiles that straddle chunks with different prompts, and query
    tiles that lie wholly in chunks without text."""
    return {
        "mixed": (layout_from_chunks([[200, 130, 70, 150], [90, 300]]),
                  chunk_prompts([None, 0, 0, 1, None, 1], [37, 100])),
        "all_prompts_distinct": (layout_from_chunks([[64, 64, 64, 65]]),
                                 chunk_prompts([0, 1, 2, 3], [5, 33, 64, 1])),
        "long_clean_prefix": (layout_from_chunks([[400, 100]]), chunk_prompts([None, 0], [300])),
        "streaming": (streaming_layout(4, 3, 96), chunk_prompts([None] * 4 + [0, 0, 1], [77, 129])),
        "unsorted_shared": (layout_from_chunks([[50, 60, 70]]), chunk_prompts([1, 0, 1], [40, 25])),
    }


CASES = _cases()


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("hq,hk", [(6, 2), (3, 1), (8, 1)])
@pytest.mark.parametrize("d", [64, 128])
def test_bf16_cross_small(name, hq, hk, d):
    lay, text = CASES[name]
    log(f"bf16 cross {name} {hq}/{hk} d={d}")
    inp, tx = inputs(lay, text, hq, hk, d, "bf16", seed=hq * 10 + hk, distinct_qx=True)
    got = run_cross(lay, text, tx, tx["q_x"], hq, hk, d, "bf16", 0.09)
    rl2, mabs, lerr = compare(*got, *ref_cross(lay, text, tx, 0.09), "bf16", tol_cross(tx, 0.09))
    log(f"  rel_l2={rl2:.3e} max_abs={mabs:.3e} lse_err={lerr:.3e}")


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("d", [64, 128])
def test_fp32_cross_small(name, d):
    lay, text = CASES[name]
    log(f"fp32 cross {name} d={d}")
    inp, tx = inputs(lay, text, 4, 2, d, "fp32", seed=d, distinct_qx=True)
    got = run_cross(lay, text, tx, tx["q_x"], 4, 2, d, "fp32", 1 / math.sqrt(d))
    compare(*got, *ref_cross(lay, text, tx, 1 / math.sqrt(d)), "fp32")


@pytest.mark.parametrize("name", list(CASES))
@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 64)])
def test_parallel_small(name, dtype, d):
    """Both attentions of one parallel launch against their oracles, with a
    cross-attention query distinct from the self-attention query and its own
    gains and temperature."""
    lay, text = CASES[name]
    log(f"parallel {name} {dtype} d={d}")
    inp, tx = inputs(lay, text, 6, 2, d, dtype, seed=7, distinct_qx=True)
    sc, scx = 1 / math.sqrt(d), 0.8 / math.sqrt(d)
    out, lse, out_x, lse_x = run_parallel(lay, text, inp, tx, 6, 2, d, dtype, sc, scx)
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    compare(out, lse, *ref, dtype)
    compare(out_x, lse_x, *ref_cross(lay, text, tx, scx), dtype, tol_cross(tx, scx))


def test_parallel_shares_the_query():
    """q_x omitted: the cross-attention reads the self-attention's q."""
    lay, text = CASES["mixed"]
    inp, tx = inputs(lay, text, 6, 2, 128, "bf16", seed=8, distinct_qx=False)
    out, lse, out_x, lse_x = run_parallel(lay, text, inp, tx, 6, 2, 128, "bf16", 0.088, 0.088, same_q=True)
    compare(out_x, lse_x, *ref_cross(lay, text, tx, 0.088), "bf16", tol_cross(tx, 0.088))


def test_parallel_equals_separate_plans_bitwise():
    """One parallel launch gives bit for bit what a self plan and a cross plan
    give separately: the work items and their arithmetic are the same, only
    the launch differs."""
    from block_causal_attention_flash_amd import Plan
    lay, text = CASES["mixed"]
    inp, tx = inputs(lay, text, 6, 2, 128, "bf16", seed=9, distinct_qx=True)
    out, lse, out_x, lse_x = run_parallel(lay, text, inp, tx, 6, 2, 128, "bf16", 0.088, 0.07)
    plan = Plan.from_layout(lay, 6, 2, 128, "bf16")
    so, sl = plan(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV), inp["q_gain"].to(DEV),
                  inp["k_gain"].to(DEV), 1e-6, 0.088)
    torch.cuda.synchronize()
    plan.close()
    xo, xl = run_cross(lay, text, tx, tx["q_x"], 6, 2, 128, "bf16", 0.07)
    assert np.array_equal(out, np64(so)) and np.array_equal(lse, np64(sl))
    assert np.array_equal(out_x, xo) and np.array_equal(lse_x, xl)


@pytest.mark.parametrize("d", [64, 128])
def test_parallel_with_split_self_attention(d):
    """A layout with too few self-attention items for the GPU: the self phase
    is split along the keys and merged, while the cross phase has chunks
    without text (merge entries without pieces) -- both in one launch."""
    from block_causal_attention_flash_amd import magi_attn_cross_plan_stats
    kv = [512 * i for i in range(17)] + [8192 + 2048, 8192 + 4096]
    q = [0] * 17 + [96, 192]
    lay = Layout(tuple(q), tuple(kv), (0, 18))
    text = chunk_prompts([None] * 17 + [0, None], [70])
    st = magi_attn_cross_plan_stats(lay.q_offsets, text.begin, text.end, text.t_text, lay.kv_offsets,
                                    lay.seq_chunks, 6, 2, d, "bf16", with_self=True)
    log(f"parallel split d={d}: {st['n_items']} workgroups")
    inp, tx = inputs(lay, text, 6, 2, d, "bf16", seed=11, distinct_qx=True)
    out, lse, out_x, lse_x = run_parallel(lay, text, inp, tx, 6, 2, d, "bf16", 0.088, 0.088)
    compare(out, lse, *oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.088,
                                        lay), "bf16")
    compare(out_x, lse_x, *ref_cross(lay, text, tx, 0.088), "bf16", tol_cross(tx, 0.088))


@pytest.mark.parametrize("online", ["cross", "self"])
def test_parallel_with_one_phase_on_the_online_softmax(online):
    """One phase's gains make the logit bound of its items large (a gain of 40
    on channel 0 of q and k, with that channel of k zero so the logits do not
    change): its workgroups run the online-softmax instance of the kernel,
    the other phase's the static one, in the same parallel launch."""
    lay, text = CASES["mixed"]
    inp, tx = inputs(lay, text, 6, 2, 128, "bf16", seed=13, distinct_qx=True)
    if online == "cross":
        tx["q_gain_x"][0] = 40.0
        tx["k_gain_x"][0] = 40.0
        tx["k_x"][:, :, 0] = 0.0
    else:
        inp["q_gain"][0] = 40.0
        inp["k_gain"][0] = 40.0
        inp["k"][:, :, 0] = 0.0
    out, lse, out_x, lse_x = run_parallel(lay, text, inp, tx, 6, 2, 128, "bf16", 0.088, 0.07)
    compare(out, lse, *oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, 0.088,
                                        lay), "bf16")
    compare(out_x, lse_x, *ref_cross(lay, text, tx, 0.07), "bf16", tol_cross(tx, 0.07))


@pytest.mark.parametrize("dtype,d", [("bf16", 128), ("bf16", 64), ("fp32", 128)])
def test_cross_without_any_text(dtype, d):
    """No chunk has text: nothing but zero rows, out = 0 and lse = -inf
    everywhere (outputs start as NaN so every row must be written)."""
    from block_causal_attention_flash_amd import CrossPlan
    lay = layout_from_chunks([[100, 29], [300]])
    text = chunk_prompts([None, None, None], [])
    plan = CrossPlan.from_layout(lay, text, 4, 2, d, dtype)
    tdt = torch.bfloat16 if dtype == "bf16" else torch.float32
    q = torch.randn(lay.t_q, 4, d, device=DEV).to(tdt)
    kx = torch.zeros(0, 2, d, device=DEV, dtype=tdt)
    out = torch.full_like(q, float("nan"))
    lse = torch.full((4, lay.t_q), float("nan"), device=DEV)
    plan(q, kx, kx, out=out, lse=lse)
    torch.cuda.synchronize()
    plan.close()
    assert torch.all(out == 0) and torch.all(torch.isneginf(lse))


# ------------------------------------------------------------------ full-size workloads, sampled rows

def sample_rows(lay, text, n_random, seed):
    rng = np.random.default_rng(seed)
    rows = set()
    for c in range(lay.n_chunks):
        a, b = lay.q_offsets[c], lay.q_offsets[c + 1]
        for r in (a, a + 1, b - 2, b - 1):
            if a <= r < b:
                rows.add(r)
    rows.update(int(x) for x in rng.integers(0, lay.t_q, n_random))
    return np.array(sorted(rows))


@pytest.mark.parametrize("name", [c.name for c in CONFIGS])
def test_parallel_workload_full_size_sampled_rows(name):
    """Each workload's parallel launch (its layout and its chunk-wise
    prompts) at full size: sampled rows of the cross-attention against the
    oracle, and a few rows of the self-attention."""
    c = get_config(name)
    lay, text = c.layout, text_layout(c)
    log(f"parallel {name}: T_q={lay.t_q} T_text={text.t_text}: generating inputs")
    inp = make_inputs(lay, c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype, c.gain_kind, c.seed)
    tx = make_text_inputs(text, c.n_kv_heads, c.head_dim, c.dtype, c.gain_kind, c.seed + 100)
    tx["q_x"] = inp["q"]
    log(f"parallel {name}: GPU run")
    out, lse, out_x, lse_x = run_parallel(lay, text, inp, tx, c.n_q_heads, c.n_kv_heads, c.head_dim, c.dtype,
                                          c.scale, c.scale, same_q=True)
    rows = np.arange(lay.t_q) if lay.t_q <= 512 else sample_rows(lay, text, 64, seed=c.seed)
    log(f"parallel {name}: cross oracle on {len(rows)} rows")
    rl2, mabs, lerr = compare(out_x[rows], lse_x[:, rows], *ref_cross(lay, text, tx, c.scale, rows), c.dtype,
                              tol_cross(tx, c.scale, rows))
    log(f"parallel {name}: cross rows={len(rows)} rel_l2={rl2:.3e} max_abs={mabs:.3e} lse_err={lerr:.3e}")
    srows = rows if lay.t_q <= 512 else np.random.default_rng(3).choice(rows, 6, replace=False)
    srows.sort()
    ref = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], c.eps, c.scale, lay,
                           rows=srows)
    rl2, mabs, lerr = compare(out[srows], lse[:, srows], *ref, c.dtype)
    log(f"parallel {name}: self rows={len(srows)} rel_l2={rl2:.3e} max_abs={mabs:.3e} lse_err={lerr:.3e}")
