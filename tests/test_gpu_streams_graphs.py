"""Streams and HIP graphs through the C ABI.

* The forward, the parallel forward and the backward enqueue only kernel
  launches on the caller's stream (no allocation, memset or synchronisation),
  so a caller can capture them into a graph, as the pages' inference stack does
  with CUDA Graphs to cut per-step launch latency (paperlayer §4.2.1;
  paper-notes §3.8, time to first chunk 3.00 s -> 2.30 s). The captured graph is
  replayed several times, with the program's own eager work and
  synchronisations between replays, and every replay must equal the eager
  call bit for bit, also after new inputs are copied into the captured
  buffers.
* The Python wrappers allocate their temporaries (workspace, default gains and
  outputs) on the stream they are given, so a call on a side stream stays
  correct while the current stream allocates and writes memory meanwhile.
"""
import math
import sys

import numpy as np
import pytest
import torch

from workloads import TextLayout, layout_from_chunks, make_inputs, make_text_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return built_lib


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


LAY = layout_from_chunks([[300, 157, 91], [200, 64]])     # two videos, ragged chunks
HQ, HK, D = 6, 2, 128
SC = 1.0 / math.sqrt(D)


def _inputs(seed, gains="uniform", d=D):
    return {n: t.to(DEV) for n, t in make_inputs(LAY, HQ, HK, d, "bf16", gains, seed).items()}


def _replay_checks(graph, static, fresh, eager_fn, outs, n=3):
    """Replays `graph` n times; before replays 1.., copies the next input set
    into the captured buffers. Every replay must equal eager_fn(inputs)."""
    for r in range(n):
        src = fresh[r % len(fresh)]
        for name, t in src.items():
            static[name].copy_(t)
        torch.cuda.synchronize()
        junk = torch.randn(1 << 20, device=DEV) * 3.0          # eager work between replays
        graph.replay()
        junk.mul_(2.0)
        torch.cuda.synchronize()
        want = eager_fn(src)
        for got_t, want_t in zip(outs, want):
            assert torch.equal(got_t, want_t), f"replay {r} differs from the eager call"
        del junk


@pytest.mark.parametrize("d", [128, 64])
def test_graph_capture_forward(d):
    from block_causal_attention_flash_amd import Plan
    sc = 1.0 / math.sqrt(d)
    plan = Plan.from_layout(LAY, HQ, HK, d, "bf16")
    sets = [_inputs(s, d=d) for s in (1, 2, 3)]
    static = {n: t.clone() for n, t in sets[0].items()}
    ws = torch.empty(max(plan.workspace_size(), 16), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(static["q"])
    lse = torch.empty((HQ, LAY.t_q), dtype=torch.float32, device=DEV)

    def eager(src):
        o, l_ = plan(src["q"], src["k"], src["v"], src["q_gain"], src["k_gain"], 1e-6, sc)
        torch.cuda.synchronize()
        return o, l_

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):                          # warm-up on the capture stream
        plan(static["q"], static["k"], static["v"], static["q_gain"], static["k_gain"], 1e-6, sc, out=out, lse=lse,
             workspace=ws, stream=s)
    torch.cuda.current_stream().wait_stream(s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan(static["q"], static["k"], static["v"], static["q_gain"], static["k_gain"], 1e-6, sc, out=out, lse=lse,
             workspace=ws, stream=s)
    _replay_checks(g, static, sets, eager, (out, lse))
    log(f"graph forward d={d}: 3 replays equal the eager calls")
    plan.close()


def test_graph_capture_forward_online_fallback():
    """Gains that send every item to the running-maximum instance (a gain of
    40 on channel 0 of q and k, with k zero there): both instances and the
    flags between them live inside the graph."""
    from block_causal_attention_flash_amd import Plan
    plan = Plan.from_layout(LAY, HQ, HK, D, "bf16")
    sets = []
    for sd in (4, 5):
        x = _inputs(sd)
        x["q_gain"][0] = 40.0
        x["k_gain"][0] = 40.0
        x["k"][:, :, 0] = 0.0
        sets.append(x)
    static = {n: t.clone() for n, t in sets[0].items()}
    ws = torch.empty(max(plan.workspace_size(), 16), dtype=torch.uint8, device=DEV)
    out = torch.empty_like(static["q"])
    lse = torch.empty((HQ, LAY.t_q), dtype=torch.float32, device=DEV)

    def eager(src):
        o, l_ = plan(src["q"], src["k"], src["v"], src["q_gain"], src["k_gain"], 1e-6, SC)
        torch.cuda.synchronize()
        return o, l_

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    plan(static["q"], static["k"], static["v"], static["q_gain"], static["k_gain"], 1e-6, SC, out=out, lse=lse,
         workspace=ws, stream=s)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        plan(static["q"], static["k"], static["v"], static["q_gain"], static["k_gain"], 1e-6, SC, out=out, lse=lse,
             workspace=ws, stream=s)
    _replay_checks(g, static, sets, eager, (out, lse))
    plan.close()


def test_graph_capture_parallel_forward():
    from block_causal_attention_flash_amd import ParallelPlan
    # chunk 0 and 3 clean, one prompt shared by chunks 1 and 2, one for chunk 4
    text = TextLayout((0, 0, 0, 40, 40), (0, 40, 40, 40, 107), 107)
    plan = ParallelPlan.from_layout(LAY, text, HQ, HK, D, "bf16")
    sets = []
    for sd in (6, 7):
        x = _inputs(sd)
        tx = make_text_inputs(text, HK, D, "bf16", "uniform", sd + 50)
        x.update({n: t.to(DEV) for n, t in tx.items()})
        x["q_x"] = (x["q"] * 0.5).contiguous()
        sets.append(x)
    static = {n: t.clone() for n, t in sets[0].items()}
    ws = torch.empty(max(plan.workspace_size(), 16), dtype=torch.uint8, device=DEV)
    bufs = [torch.empty_like(static["q"]), torch.empty((HQ, LAY.t_q), dtype=torch.float32, device=DEV),
            torch.empty_like(static["q"]), torch.empty((HQ, LAY.t_q), dtype=torch.float32, device=DEV)]

    def call(src, stream=None, outs=None, workspace=None):
        kw = {} if outs is None else dict(out=outs[0], lse=outs[1], out_x=outs[2], lse_x=outs[3])
        return plan(src["q"], src["k"], src["v"], src["k_x"], src["v_x"], q_x=src["q_x"], q_gain=src["q_gain"],
                    k_gain=src["k_gain"], q_gain_x=src["q_gain_x"], k_gain_x=src["k_gain_x"], rms_eps=1e-6,
                    scale=SC, scale_x=0.8 * SC, workspace=workspace, stream=stream, **kw)

    def eager(src):
        r = call(src)
        torch.cuda.synchronize()
        return r

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    call(static, stream=s, outs=bufs, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(static, stream=s, outs=bufs, workspace=ws)
    _replay_checks(g, static, sets, eager, bufs)
    log("graph parallel forward: replays equal the eager calls")
    plan.close()


@pytest.mark.parametrize("d", [128, 64])
def test_graph_capture_backward(d):
    from block_causal_attention_flash_amd import TrainPlan
    sc = 1.0 / math.sqrt(d)
    plan = TrainPlan.from_layout(LAY, HQ, HK, d, "bf16")
    sets = []
    for sd in (8, 9):
        x = _inputs(sd, d=d)
        o, l_ = plan(x["q"], x["k"], x["v"], x["q_gain"], x["k_gain"], 1e-6, sc)
        x["out"], x["lse"] = o, l_
        x["dout"] = torch.from_numpy(np.random.default_rng(sd).standard_normal((LAY.t_q, HQ, d)).astype(
            np.float32)).to(torch.bfloat16).to(DEV)
        sets.append(x)
    torch.cuda.synchronize()
    static = {n: t.clone() for n, t in sets[0].items()}
    ws = torch.empty(max(plan.bwd_workspace_size(), 16), dtype=torch.uint8, device=DEV)
    grads = [torch.empty_like(static["q"]), torch.empty_like(static["k"]), torch.empty_like(static["v"]),
             torch.empty(d, dtype=torch.float32, device=DEV), torch.empty(d, dtype=torch.float32, device=DEV)]

    def call(src, stream=None, outs=None, workspace=None):
        kw = {} if outs is None else dict(dq=outs[0], dk=outs[1], dv=outs[2], dq_gain=outs[3], dk_gain=outs[4])
        return plan.backward(src["q"], src["k"], src["v"], src["out"], src["lse"], src["dout"], src["q_gain"],
                             src["k_gain"], 1e-6, sc, workspace=workspace, stream=stream, **kw)

    def eager(src):
        r = call(src)
        torch.cuda.synchronize()
        return r

    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    call(static, stream=s, outs=grads, workspace=ws)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=s):
        call(static, stream=s, outs=grads, workspace=ws)
    _replay_checks(g, static, sets, eager, grads)
    log(f"graph backward d={d}: replays equal the eager calls")
    plan.close()


def test_side_stream_with_default_temporaries():
    """Forward and backward on a side stream behind a long matrix product,
    with the workspace, gains and outputs allocated by the wrappers. The
    current stream then allocates and overwrites memory while the side stream
    still works; the results must equal the current-stream calls bit for
    bit."""
    from block_causal_attention_flash_amd import TrainPlan
    plan = TrainPlan.from_layout(LAY, HQ, HK, D, "bf16")
    x = _inputs(10)
    dout = torch.from_numpy(np.random.default_rng(10).standard_normal((LAY.t_q, HQ, D)).astype(np.float32)).to(
        torch.bfloat16).to(DEV)
    side = torch.cuda.Stream()
    for trial in range(3):
        side.wait_stream(torch.cuda.current_stream())
        with torch.cuda.stream(side):
            a = torch.randn(4096, 4096, device=DEV)
            for _ in range(8):
                a = a @ a.T * 1e-2                          # keeps the side stream busy
        o, l_ = plan(x["q"], x["k"], x["v"], None, None, 1e-6, SC, stream=side)
        gr = plan.backward(x["q"], x["k"], x["v"], o, l_, dout, None, None, 1e-6, SC, stream=side)
        junk = [torch.full((1 << 22,), float(i + 1), device=DEV) for i in range(16)]   # current stream
        del junk
        torch.cuda.synchronize()
        ro, rl = plan(x["q"], x["k"], x["v"], torch.ones(D, device=DEV), torch.ones(D, device=DEV), 1e-6, SC)
        rg = plan.backward(x["q"], x["k"], x["v"], ro, rl, dout, torch.ones(D, device=DEV), torch.ones(D, device=DEV),
                           1e-6, SC)
        torch.cuda.synchronize()
        assert torch.equal(o, ro) and torch.equal(l_, rl), trial
        for a_, b_ in zip(gr, rg):
            assert torch.equal(a_, b_), trial
    plan.close()
