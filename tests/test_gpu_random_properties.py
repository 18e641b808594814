"""Exact properties over seeded random layouts, checked without the oracle
(so the layouts can be wider than the oracle-compared ones): chunks of up to
300 tokens, up to three packed videos with cached leading chunks, KV ranges,
last global blocks, chunk-wise prompts, and head shapes from MHA to 48/8.

- One parallel launch (self- and cross-attention as phases of one kernel)
  equals a self plan and a cross plan run separately, bit for bit: the work
  items and their arithmetic are the same, only the launch differs.
- The backward of a self and of a cross training plan is deterministic: a
  second call gives the same bits (fixed-order reductions, split lists merged
  in piece order).
"""
import math
import sys

import numpy as np
import pytest
import torch

from workloads import Layout, TextLayout

pytestmark = pytest.mark.gpu

DEV = "cuda:0"
SEEDS = list(range(40))
HEADS = [(2, 1), (4, 2), (6, 2), (3, 3), (8, 1), (12, 4), (16, 2), (24, 8), (16, 16), (32, 4), (48, 8)]


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return built_lib


def wide_case(seed):
    """A layout, a chunk-wise text for it and a head shape from default_rng."""
    rng = np.random.default_rng(77000 + seed)
    q_off, kv_off, seq = [0], [0], [0]
    for _ in range(int(rng.integers(1, 4))):
        n_ch = int(rng.integers(1, 5))
        n_cached = int(rng.integers(0, n_ch))
        for c in range(n_ch):
            kv_off.append(kv_off[-1] + int(rng.integers(1, 300)))
            q_off.append(q_off[-1] + (0 if c < n_cached else int(rng.integers(1, 300))))
        seq.append(seq[-1] + n_ch)
    lay = Layout(tuple(q_off), tuple(kv_off), tuple(seq), kv_range=int(rng.choice([0, 0, 1, 2, 3])),
                 last_global=int(rng.integers(0, 2)))
    # per video: leading clean chunks, then that video's prompts, each shared by a run of adjacent chunks
    lengths = [int(x) for x in rng.integers(1, 300, 2 * (len(seq) - 1))]
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
    hq, hk = HEADS[int(rng.integers(0, len(HEADS)))]
    return lay, text, hq, hk


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


@pytest.mark.parametrize("seed", SEEDS)
def test_parallel_launch_equals_separate_plans(seed):
    from block_causal_attention_flash_amd import Plan
    from test_gpu_cross import inputs, np64, run_cross, run_parallel
    lay, text, hq, hk = wide_case(seed)
    log(f"parallel {seed}: t_q {lay.t_q} t_k {lay.t_k} t_text {text.t_text} heads {hq}/{hk}")
    inp, tx = inputs(lay, text, hq, hk, 128, "bf16", seed=seed, distinct_qx=True)
    out, lse, out_x, lse_x = run_parallel(lay, text, inp, tx, hq, hk, 128, "bf16", 0.088, 0.07)
    plan = Plan.from_layout(lay, hq, hk, 128, "bf16")
    so, sl = plan(inp["q"].to(DEV), inp["k"].to(DEV), inp["v"].to(DEV), inp["q_gain"].to(DEV),
                  inp["k_gain"].to(DEV), 1e-6, 0.088)
    torch.cuda.synchronize()
    so, sl = np64(so), np64(sl)
    plan.close()
    xo, xl = run_cross(lay, text, tx, tx["q_x"], hq, hk, 128, "bf16", 0.07)
    assert np.array_equal(out, so) and np.array_equal(lse, sl)
    assert np.array_equal(out_x, xo) and np.array_equal(lse_x, xl)


@pytest.mark.parametrize("seed", SEEDS)
def test_backward_is_deterministic(seed):
    from block_causal_attention_flash_amd import CrossTrainPlan, TrainPlan
    from test_gpu_cross import inputs
    lay, text, hq, hk = wide_case(seed)
    log(f"determinism {seed}: t_q {lay.t_q} t_k {lay.t_k} t_text {text.t_text} heads {hq}/{hk}")
    inp, tx = inputs(lay, text, hq, hk, 128, "bf16", seed=seed, distinct_qx=True)
    g = {k: t.to(DEV) for k, t in inp.items()}
    gx = {k: t.to(DEV) for k, t in tx.items()}
    dout = torch.randn(lay.t_q, hq, 128, generator=torch.Generator().manual_seed(seed)).to(torch.bfloat16).to(DEV)
    sc = 1 / math.sqrt(128)
    for plan, args in ((TrainPlan.from_layout(lay, hq, hk, 128, "bf16"),
                        (g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"])),
                       (CrossTrainPlan.from_layout(lay, text, hq, hk, 128, "bf16"),
                        (gx["q_x"], gx["k_x"], gx["v_x"], gx["q_gain_x"], gx["k_gain_x"]))):
        out, lse = plan(*args, 1e-6, sc)
        first = [t.clone() for t in plan.backward(*args[:3], out, lse, dout, *args[3:], 1e-6, sc)]
        second = plan.backward(*args[:3], out, lse, dout, *args[3:], 1e-6, sc)
        torch.cuda.synchronize()
        plan.close()
        for a, b in zip(first, second):
            assert torch.equal(a, b)
