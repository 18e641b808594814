"""Seeded random layouts through the whole path (C ABI): the forward and the
backward of a training plan against the fp64 oracle, and, for a random text,
the cross-attention's forward and backward.

Each layout mixes what the fixed cases test one at a time: packed videos of
one to three chunks, ragged chunk lengths off the tile grids, leading cached
chunks without queries (a KV cache), a KV-range window, a last global block,
and several GQA ratios. Tolerances are those of the fixed cases: forward bf16
max-abs 2e-2 and relative L2 5e-3; backward relative L2 1e-2 per gradient. The
LSE is held to 1e-2 on rows that see at least 8 keys. A row that sees fewer
has nearly one logit as its LSE, so that logit's bf16 rounding shows undamped:
such rows take the larger of 1e-2 and five times the largest RMS logit error
of their keys under the bf16 error model (tests/bf16_error_model.py, pinned on
the CPU).
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from bf16_error_model import lse_tolerance
from workloads import Layout, TextLayout, make_inputs, make_text_inputs

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SEEDS = list(range(30))


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import block_causal_attention_flash_amd  # noqa: F401
    return built_lib


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def random_case(seed):
    """A layout, a text for it and a head configuration from default_rng(seed)."""
    rng = np.random.default_rng(1000 + seed)
    q_off, kv_off, seq = [0], [0], [0]
    for _ in range(int(rng.integers(1, 4))):
        n_ch = int(rng.integers(1, 5))
        n_cached = int(rng.integers(0, n_ch))           # leading chunks without queries
        for c in range(n_ch):
            kv_off.append(kv_off[-1] + int(rng.integers(1, 170)))
            q_off.append(q_off[-1] + (0 if c < n_cached else int(rng.integers(1, 170))))
        seq.append(seq[-1] + n_ch)
    lay = Layout(tuple(q_off), tuple(kv_off), tuple(seq), kv_range=int(rng.choice([0, 0, 1, 2, 3])),
                 last_global=int(rng.integers(0, 2)))
    # text: per video, leading clean chunks without text, then prompts of
    # that video, each shared by a run of adjacent chunks (one run of rows
    # per prompt, as chunk-wise prompts give)
    lengths = [int(x) for x in rng.integers(1, 90, 2 * (len(seq) - 1))]
    starts = np.concatenate([[0], np.cumsum(lengths)])
    begin, end = [], []
    for v in range(len(seq) - 1):
        n_clean = int(rng.integers(0, 2))
        cur = 2 * v
        for c in range(seq[v], seq[v + 1]):
            if c - seq[v] < n_clean:
                begin.append(0)
                end.append(0)
                continue
            if c - seq[v] > n_clean and cur == 2 * v and rng.random() < 0.4:
                cur += 1
            begin.append(int(starts[cur]))
            end.append(int(starts[cur + 1]))
    text = TextLayout(tuple(begin), tuple(end), int(starts[-1]))
    hq, hk = [(2, 1), (4, 2), (6, 2), (3, 3), (8, 1)][seed % 5]
    return lay, text, hq, hk


def rows_and_keys(lay, text=None):
    """Rows that see no key and keys no row sees (from the layout, or the
    text for the cross-attention): the places the gradient must be exactly 0."""
    import oracle as orc
    if text is None:
        m = orc.block_causal_mask(lay)
    else:
        m = orc.text_mask(lay.q_offsets, text)
    return ~m.any(axis=1), ~m.any(axis=0)


def lse_tol(q, k, q_gain, k_gain, scale, mask):
    """[H, T] LSE tolerance (bf16_error_model.lse_tolerance): 1e-2 for rows
    that see at least 8 keys; for rows with fewer, the larger of 1e-2 and five
    times the largest RMS logit error the bf16 operand rounding gives among
    the row's keys."""
    return lse_tolerance(q, k, q_gain, k_gain, 1e-6, scale, mask)


def rel_l2(got, ref):
    n = np.linalg.norm(ref)
    return float(np.linalg.norm(got - ref) / n) if n > 0 else float(np.linalg.norm(got))


def head_dim_of(seed):
    """bf16 head_dim of a random case: 64 on every third seed, else 128."""
    return 64 if seed % 3 == 0 else 128


def describe(lay, text, hq, hk):
    return (f"q_offsets={lay.q_offsets} kv_offsets={lay.kv_offsets} seq_chunks={lay.seq_chunks} "
            f"kv_range={lay.kv_range} last_global={lay.last_global} text={text.begin}/{text.end}/{text.t_text} "
            f"heads={hq}/{hk}")


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layout_self_attention(seed):
    from block_causal_attention_flash_amd import TrainPlan
    lay, text, hq, hk = random_case(seed)
    hd = head_dim_of(seed)
    log(f"random self {seed}: {describe(lay, text, hq, hk)} d={hd}")
    sc = 1 / math.sqrt(hd)
    inp = make_inputs(lay, hq, hk, hd, "bf16", "uniform", seed)
    dout = torch.from_numpy(np.random.default_rng(seed + 7).standard_normal((lay.t_q, hq, hd))
                            .astype(np.float32)).to(torch.bfloat16)
    g = {n: t.to(DEV) for n, t in inp.items()}
    plan = TrainPlan.from_layout(lay, hq, hk, hd, "bf16")
    out, lse = plan(g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], 1e-6, sc)
    dq, dk, dv = (torch.full_like(g[n], float("nan")) for n in ("q", "k", "v"))
    grads = plan.backward(g["q"], g["k"], g["v"], out, lse, dout.to(DEV), g["q_gain"], g["k_gain"], 1e-6, sc,
                          dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    got_out, got_lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
    got = [t.double().cpu().numpy() for t in grads]
    plan.close()
    ref_out, ref_lse = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    d = got_out - ref_out
    assert np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_lse))
    assert np.max(np.abs(d)) <= 2e-2 and rel_l2(got_out, ref_out) <= 5e-3
    assert np.all(np.abs(got_lse - ref_lse) <= lse_tol(inp["q"], inp["k"], inp["q_gain"], inp["k_gain"], sc,
                                                        oracle.block_causal_mask(lay)))
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay,
                                    dout)
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    for a in got:
        assert np.all(np.isfinite(a))
    assert max(errs) <= 1e-2, dict(zip(("dq", "dk", "dv", "dq_gain", "dk_gain"), errs))
    _, unseen = rows_and_keys(lay)
    assert np.all(got[1][unseen] == 0) and np.all(got[2][unseen] == 0)


@pytest.mark.parametrize("seed", SEEDS)
def test_random_layout_cross_attention(seed):
    lay, text, hq, hk = random_case(seed)
    log(f"random cross {seed}: {describe(lay, text, hq, hk)}")
    check_cross(seed, lay, text, hq, hk)


def check_cross(seed, lay, text, hq, hk):
    from block_causal_attention_flash_amd import CrossTrainPlan
    hd = head_dim_of(seed)
    sc = 0.8 / math.sqrt(hd)
    q = make_inputs(lay, hq, hk, hd, "bf16", "uniform", seed)["q"]
    tx = make_text_inputs(text, hk, hd, "bf16", "uniform", seed + 1)
    dout = torch.from_numpy(np.random.default_rng(seed + 9).standard_normal((lay.t_q, hq, hd))
                            .astype(np.float32)).to(torch.bfloat16)
    g = {n: t.to(DEV) for n, t in tx.items()}
    plan = CrossTrainPlan.from_layout(lay, text, hq, hk, hd, "bf16")
    out, lse = plan(q.to(DEV), g["k_x"], g["v_x"], g["q_gain_x"], g["k_gain_x"], 1e-6, sc)
    dq = torch.full_like(q.to(DEV), float("nan"))
    dk, dv = (torch.full_like(g[n], float("nan")) for n in ("k_x", "v_x"))
    grads = plan.backward(q.to(DEV), g["k_x"], g["v_x"], out, lse, dout.to(DEV), g["q_gain_x"], g["k_gain_x"], 1e-6,
                          sc, dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    got_out, got_lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
    got = [t.double().cpu().numpy() for t in grads]
    plan.close()
    ref_out, ref_lse = oracle.cross_attention(q, tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, sc,
                                              lay.q_offsets, text)
    assert np.all(np.isfinite(got_out))
    assert np.max(np.abs(got_out - ref_out)) <= 2e-2 and rel_l2(got_out, ref_out) <= 5e-3
    live = np.isfinite(ref_lse)
    assert np.array_equal(np.isfinite(got_lse), live) and np.all(got_out[~live.T.any(axis=1)] == 0)
    bound = lse_tol(q, tx["k_x"], tx["q_gain_x"], tx["k_gain_x"], sc, oracle.text_mask(lay.q_offsets, text))
    assert np.all(np.abs(got_lse[live] - ref_lse[live]) <= bound[live])
    ref = oracle.cross_attention_backward(q, tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, sc,
                                          lay.q_offsets, text, dout)
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    for a in got:
        assert np.all(np.isfinite(a))
    assert max(errs) <= 1e-2, dict(zip(("dq", "dk", "dv", "dq_gain", "dk_gain"), errs))
    no_text, unseen = rows_and_keys(lay, text)
    assert np.all(got[0][no_text] == 0)
    assert np.all(got[1][unseen] == 0) and np.all(got[2][unseen] == 0)


@pytest.mark.parametrize("seed", SEEDS[:10])
def test_random_layout_fp32(seed):
    """The fp32 path (d = 64 on even seeds, 128 on odd ones): forward and
    backward of the self- and the cross-attention at relative 1e-5."""
    from block_causal_attention_flash_amd import CrossTrainPlan, TrainPlan
    lay, text, hq, hk = random_case(seed)
    d = 64 if seed % 2 == 0 else 128
    log(f"random fp32 {seed} d={d}: {describe(lay, text, hq, hk)}")
    sc = 1 / math.sqrt(d)
    inp = make_inputs(lay, hq, hk, d, "fp32", "uniform", seed)
    tx = make_text_inputs(text, hk, d, "fp32", "uniform", seed + 1)
    dout = torch.from_numpy(np.random.default_rng(seed + 7).standard_normal((lay.t_q, hq, d)).astype(np.float32))
    cases = [(TrainPlan.from_layout(lay, hq, hk, d, "fp32"), inp["k"], inp["v"], inp["q_gain"], inp["k_gain"],
              lambda: oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay),
              lambda: oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc,
                                                lay, dout)),
             (CrossTrainPlan.from_layout(lay, text, hq, hk, d, "fp32"), tx["k_x"], tx["v_x"], tx["q_gain_x"],
              tx["k_gain_x"],
              lambda: oracle.cross_attention(inp["q"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], 1e-6, sc,
                                             lay.q_offsets, text),
              lambda: oracle.cross_attention_backward(inp["q"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"],
                                                      1e-6, sc, lay.q_offsets, text, dout))]
    for plan, k, v, gq, gk, fwd_ref, bwd_ref in cases:
        q, k, v, gq, gk = (t.to(DEV) for t in (inp["q"], k, v, gq, gk))
        out, lse = plan(q, k, v, gq, gk, 1e-6, sc)
        dq, dk, dv = (torch.full_like(t, float("nan")) for t in (q, k, v))
        grads = plan.backward(q, k, v, out, lse, dout.to(DEV), gq, gk, 1e-6, sc, dq=dq, dk=dk, dv=dv)
        torch.cuda.synchronize()
        got_out, got_lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
        got = [t.double().cpu().numpy() for t in grads]
        plan.close()
        ref_out, ref_lse = fwd_ref()
        assert rel_l2(got_out, ref_out) <= 1e-5
        live = np.isfinite(ref_lse)
        assert np.array_equal(np.isfinite(got_lse), live)
        assert np.max(np.abs(got_lse[live] - ref_lse[live]), initial=0.0) <= 1e-5
        errs = [rel_l2(a, b) for a, b in zip(got, bwd_ref())]
        for a in got:
            assert np.all(np.isfinite(a))
        assert max(errs) <= 1e-5, dict(zip(("dq", "dk", "dv", "dq_gain", "dk_gain"), errs))


@pytest.mark.parametrize("seed,hq,hk", [(3, 24, 2), (5, 32, 2), (7, 24, 1), (9, 32, 1), (11, 48, 1)])
def test_random_layout_wide_groups(seed, hq, hk):
    """Query-head groups of 12, 16, 24, 32 and 48 (forward work items of 32
    down to 8 tokens of every head of the group; backward items of at least
    32 tokens): forward and backward against the oracle."""
    from block_causal_attention_flash_amd import TrainPlan
    lay, _, _, _ = random_case(seed)
    log(f"random wide groups {seed} {hq}/{hk}: {lay}")
    sc = 1 / math.sqrt(128)
    inp = make_inputs(lay, hq, hk, 128, "bf16", "uniform", seed)
    dout = torch.from_numpy(np.random.default_rng(seed + 7).standard_normal((lay.t_q, hq, 128))
                            .astype(np.float32)).to(torch.bfloat16)
    g = {n: t.to(DEV) for n, t in inp.items()}
    plan = TrainPlan.from_layout(lay, hq, hk, 128, "bf16")
    out, lse = plan(g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], 1e-6, sc)
    dq, dk, dv = (torch.full_like(g[n], float("nan")) for n in ("q", "k", "v"))
    grads = plan.backward(g["q"], g["k"], g["v"], out, lse, dout.to(DEV), g["q_gain"], g["k_gain"], 1e-6, sc,
                          dq=dq, dk=dk, dv=dv)
    torch.cuda.synchronize()
    got_out, got_lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
    got = [t.double().cpu().numpy() for t in grads]
    plan.close()
    ref_out, ref_lse = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    assert np.max(np.abs(got_out - ref_out)) <= 2e-2 and rel_l2(got_out, ref_out) <= 5e-3
    assert np.all(np.abs(got_lse - ref_lse) <= lse_tol(inp["q"], inp["k"], inp["q_gain"], inp["k_gain"], sc,
                                                        oracle.block_causal_mask(lay)))
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay,
                                    dout)
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    assert all(np.all(np.isfinite(a)) for a in got)
    assert max(errs) <= 1e-2, dict(zip(("dq", "dk", "dv", "dq_gain", "dk_gain"), errs))


@pytest.mark.parametrize("seed,hq,hk", [(4, 24, 2), (6, 32, 2), (8, 24, 1), (10, 48, 1)])
def test_random_layout_wide_groups_cross(seed, hq, hk):
    """The cross-attention's forward and backward with groups of 12 to 48."""
    lay, text, _, _ = random_case(seed)
    log(f"random cross wide groups {seed} {hq}/{hk}: {describe(lay, text, hq, hk)}")
    check_cross(seed, lay, text, hq, hk)



def split_cache_case(seed):
    """A KV-cache layout the plan splits: 4 to 39 cached chunks of 64 to 1,023
    keys, then 1 to 3 query chunks of up to 299 tokens, so that few work items
    hold long key lists (2 to 8 pieces each, merged afterwards)."""
    rng = np.random.default_rng(91000 + seed)
    n_cached, n_q = int(rng.integers(4, 40)), int(rng.integers(1, 4))
    kv, q = [0], [0]
    for c in range(n_cached + n_q):
        kv.append(kv[-1] + int(rng.integers(64, 1024)))
        q.append(q[-1] + (0 if c < n_cached else int(rng.integers(1, 300))))
    lay = Layout(tuple(q), tuple(kv), (0, n_cached + n_q), kv_range=int(rng.choice([0, 0, 6, 12])), last_global=0)
    hq, hk = [(2, 1), (4, 2), (6, 2), (8, 1), (12, 4), (16, 2), (24, 8)][int(rng.integers(0, 7))]
    return lay, hq, hk


@pytest.mark.parametrize("seed", list(range(6)))
def test_random_split_kv_cache(seed):
    from block_causal_attention_flash_amd import TrainPlan, magi_attn_plan_stats
    lay, hq, hk = split_cache_case(seed)
    st = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, hq, hk, 128, "bf16")
    whole = -(-lay.t_q // st["tile_q"]) * hk * (hq // hk // st["heads_per_item"])
    log(f"random split {seed}: t_q {lay.t_q} t_k {lay.t_k} heads {hq}/{hk} items {st['n_items']} of {whole}")
    assert st["n_items"] >= 2 * whole                      # every list was cut
    sc = 1 / math.sqrt(128)
    inp = make_inputs(lay, hq, hk, 128, "bf16", "uniform", seed)
    dout = torch.from_numpy(np.random.default_rng(seed + 7).standard_normal((lay.t_q, hq, 128))
                            .astype(np.float32)).to(torch.bfloat16)
    g = {n: t.to(DEV) for n, t in inp.items()}
    plan = TrainPlan.from_layout(lay, hq, hk, 128, "bf16")
    out, lse = plan(g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], 1e-6, sc)
    grads = plan.backward(g["q"], g["k"], g["v"], out, lse, dout.to(DEV), g["q_gain"], g["k_gain"], 1e-6, sc)
    torch.cuda.synchronize()
    got_out, got_lse = out.double().cpu().numpy(), lse.double().cpu().numpy()
    got = [t.double().cpu().numpy() for t in grads]
    plan.close()
    ref_out, ref_lse = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    assert np.all(np.isfinite(got_out)) and np.all(np.isfinite(got_lse))
    assert np.max(np.abs(got_out - ref_out)) <= 2e-2 and rel_l2(got_out, ref_out) <= 5e-3
    assert np.all(np.abs(got_lse - ref_lse) <= lse_tol(inp["q"], inp["k"], inp["q_gain"], inp["k_gain"], sc,
                                                        oracle.block_causal_mask(lay)))
    ref = oracle.attention_backward(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay, dout)
    errs = [rel_l2(a, b) for a, b in zip(got, ref)]
    assert max(errs) <= 1e-2, dict(zip(("dq", "dk", "dv", "dq_gain", "dk_gain"), errs))
