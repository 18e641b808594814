"""Benchmark of the block-causal attention forward on one MI355X.

python bench.py [--gpus 1] [--steps K] [--warmup W] [--workload NAME] [--kv-range R] [--last-global]
                [--attention self|cross|parallel] [--backward] [--no-cpu-baseline]

A step is one forward call (query/key RMSNorm, masked softmax attention, LSE)
over the whole workload, inputs resident in HBM: the block-causal
self-attention by default; with --attention cross the text cross-attention of
the workload's chunk-wise prompts; with --attention parallel both in one
launch (their useful FLOPs summed). The plan (tile
classification and work order) is built once per layout before timing; its
host time is reported as plan_create_ms. Prints one JSON line.

Useful FLOPs follow the MAGI-1 pages' accounting (paperlayer §B.2.1: the two
matrix products over the mask area): 4 * head_dim * n_q_heads * (allowed
query-key pairs per head).
"""
import argparse
import dataclasses
import hashlib
import json
import math
import os
import re
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "block-causal attn fwd useful TFLOP/s and % bf16 MFMA peak, 1×MI355X"
METRIC_CROSS = "text cross-attn fwd useful TFLOP/s and % bf16 MFMA peak, 1×MI355X"
METRIC_BACKWARD = "block-causal attn bwd useful TFLOP/s (2.5x fwd FLOPs) and % bf16 MFMA peak, 1×MI355X"
METRIC_CROSS_BACKWARD = "text cross-attn bwd useful TFLOP/s (2.5x fwd FLOPs) and % bf16 MFMA peak, 1×MI355X"
METRIC_PARALLEL = "parallel block-causal self- + text cross-attn fwd useful TFLOP/s and % bf16 MFMA peak, 1×MI355X"
PEAK_BF16_TFLOPS = 2500.0          # MI355X dense bf16 MFMA, published
KERNEL_SRC = os.path.join(ROOT, "block_causal_attention_flash_amd", "csrc", "fwd_bf16.hip")
BWD_KERNEL_SRC = os.path.join(ROOT, "block_causal_attention_flash_amd", "csrc", "bwd_bf16.hip")


def useful_pairs(layout) -> int:
    """Allowed (query, key) pairs per head, from the offsets: every query of
    chunk c sees keys from its video's first key (or, with a KV range R, from
    chunk c - R + 1 if later) to the end of chunk c; a last global block's
    queries see all T_k keys."""
    R = int(getattr(layout, "kv_range", 0))
    G = int(getattr(layout, "last_global", 0))
    total = 0
    for s in range(layout.n_seqs):
        c0, c1 = layout.seq_chunks[s], layout.seq_chunks[s + 1]
        for c in range(c0, c1):
            first = max(c0, c - R + 1) if R > 0 else c0
            keys = layout.kv_offsets[-1] if (G and s == layout.n_seqs - 1) else \
                layout.kv_offsets[c + 1] - layout.kv_offsets[first]
            total += (layout.q_offsets[c + 1] - layout.q_offsets[c]) * keys
    return total


def useful_text_pairs(layout, text) -> int:
    """Allowed (query, text key) pairs per head: chunk c's queries times its
    prompt's length."""
    return sum((layout.q_offsets[c + 1] - layout.q_offsets[c]) * (text.end[c] - text.begin[c])
               for c in range(layout.n_chunks))


KERNEL_HEADERS = [os.path.join(ROOT, "block_causal_attention_flash_amd", "csrc", h) for h in ("cdna4.hpp", "kernels.hpp")]


def kernel_hash(path: str = KERNEL_SRC) -> str:
    """sha256 (16 hex digits) of a kernel source followed by the shared
    headers it compiles with, comments and blank space removed, so that the
    stored counters go stale on code changes only."""
    src = ""
    for name in [path] + KERNEL_HEADERS:
        with open(name) as f:
            src += f.read() + "\n"
    src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
    src = re.sub(r"//[^\n]*", " ", src)
    src = " ".join(src.split())
    return hashlib.sha256(src.encode()).hexdigest()[:16]


def stored_traffic(workload: str, attention: str = "self"):
    """HBM bytes per launch from the committed rocprofv3 counter summary, or
    None when it is missing or was taken on a different kernel source."""
    suffix = "" if attention == "self" else f"_{attention}"
    path = os.path.join(ROOT, "profiles", f"fwd_bf16_{workload}{suffix}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("kernel_sha256_16") != kernel_hash():
        return None
    return doc.get("hbm_bytes_per_launch")


def stored_backward_traffic(workload: str):
    """HBM bytes per backward call (all of its kernels) from the committed
    counter summary, or None when missing or taken on a different source."""
    path = os.path.join(ROOT, "profiles", f"bwd_bf16_{workload}_traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        doc = json.load(f)
    if doc.get("kernel_sha256_16") != kernel_hash(BWD_KERNEL_SRC):
        return None
    return doc.get("hbm_bytes_per_call")


def first_visible(lay, c):
    """First chunk whose keys chunk c sees (its video's first, or with a KV
    range R the later of that and c - R + 1)."""
    R = int(getattr(lay, "kv_range", 0))
    s = next(i for i in range(lay.n_seqs) if lay.seq_chunks[i] <= c < lay.seq_chunks[i + 1])
    return max(lay.seq_chunks[s], c - R + 1) if R > 0 else lay.seq_chunks[s]


def timing_record(times, span, steps):
    import statistics
    return {"mean_ms": round(span / steps, 4), "median_ms": round(statistics.median(times), 4),
            "min_ms": round(min(times), 4), "max_ms": round(max(times), 4)}


def cpu_model() -> str:
    """The host CPU's model name (/proc/cpuinfo), for the baseline's record."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def step_times(step, stream, steps: int, flush=None):
    """Runs `steps` steps on `stream`, each between two HIP events recorded
    on that stream (the one the kernels are launched on); with `flush` (a
    device buffer), overwrites it before every step, outside the timed pair,
    so that each step starts with the caches holding other data. Returns the
    per-step times (ms) and the events' total span (ms, warm runs only)."""
    import torch
    evs = [torch.cuda.Event(enable_timing=True) for _ in range(2 * steps)]
    for i in range(steps):
        if flush is not None:
            flush.fill_(i & 0xff)
        evs[2 * i].record(stream)
        step()
        evs[2 * i + 1].record(stream)
    torch.cuda.synchronize()
    times = [evs[2 * i].elapsed_time(evs[2 * i + 1]) for i in range(steps)]
    span = evs[0].elapsed_time(evs[-1]) if flush is None else sum(times)
    return times, span


def cpu_baseline(cfg, inp, budget_s: float = 20.0, attention: str = "self", text=None, tx=None):
    """Times the fp64 oracle(s) of the benchmarked attention on a bounded
    sample of query rows (all heads) and converts it to useful TFLOP/s on
    those rows."""
    import numpy as np
    import oracle
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    lay = cfg.layout
    d, hq = cfg.head_dim, cfg.n_q_heads
    rng = np.random.default_rng(0)
    # row blocks of 32 consecutive tokens from randomly chosen chunks
    flops = 0.0
    spent = 0.0
    rows_done = 0
    t_start = time.perf_counter()
    qc = [c for c in range(lay.n_chunks) if lay.q_offsets[c + 1] > lay.q_offsets[c]]
    while spent < budget_s and rows_done < lay.t_q:
        c = qc[int(rng.integers(0, len(qc)))]
        a, b = lay.q_offsets[c], lay.q_offsets[c + 1]
        r0 = int(rng.integers(a, max(a + 1, b - 32)))
        rows = np.arange(r0, min(b, r0 + 32))
        t0 = time.perf_counter()
        if attention in ("self", "parallel"):
            oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], cfg.eps, cfg.scale, lay,
                             rows=rows)
            glob = lay.last_global and c >= lay.seq_chunks[-2]
            keys = lay.t_k if glob else lay.kv_offsets[c + 1] - lay.kv_offsets[first_visible(lay, c)]
            flops += 4.0 * d * hq * len(rows) * keys
        if attention in ("cross", "parallel"):
            oracle.cross_attention(inp["q"], tx["k_x"], tx["v_x"], tx["q_gain_x"], tx["k_gain_x"], cfg.eps,
                                   cfg.scale, lay.q_offsets, text, rows=rows)
            flops += 4.0 * d * hq * len(rows) * (text.end[c] - text.begin[c])
        spent += time.perf_counter() - t0
        rows_done += len(rows)
        if time.perf_counter() - t_start > 3 * budget_s:
            break
    what = {"self": "", "cross": " (cross-attention)", "parallel": " (self- and cross-attention)"}[attention]
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"{rows_done} query rows x {hq} heads of {cfg.name}{what} (blocks of 32 rows), "
                      f"{spent:.1f} s fp64 numpy on the host"}


def cpu_baseline_backward(cfg, inp, dout, budget_s: float = 20.0, text=None):
    """Times the fp64 backward oracle on a bounded sample: the first n tokens
    of the workload's first chunk (with text, for the cross-attention) as a
    one-chunk layout, n doubling from 256 while the oracle takes under a
    quarter of the budget. Useful FLOPs as the GPU line counts them: 2.5x the
    forward's over the sample's pairs."""
    import numpy as np
    import oracle
    from workloads import Layout, TextLayout
    try:
        from threadpoolctl import threadpool_info
        threads = max([p.get("num_threads", 1) for p in threadpool_info()] or [1])
    except Exception:  # pragma: no cover
        threads = 1
    lay = cfg.layout
    d, hq = cfg.head_dim, cfg.n_q_heads
    if text is None:
        c = next(c for c in range(lay.n_chunks) if lay.q_offsets[c + 1] > lay.q_offsets[c])
    else:
        c = next((c for c in range(lay.n_chunks)
                  if lay.q_offsets[c + 1] > lay.q_offsets[c] and text.end[c] > text.begin[c]), None)
        if c is None:
            return None
    a, b = lay.q_offsets[c], lay.q_offsets[c + 1]
    ka = lay.kv_offsets[c]
    n, spent, flops = 256, 0.0, 0.0
    while True:
        n = min(n, b - a, lay.kv_offsets[c + 1] - ka) if text is None else min(n, b - a)
        sub = Layout((0, n), (0, n), (0, 1))
        q, g = inp["q"][a:a + n], dout[a:a + n]
        t0 = time.perf_counter()
        if text is None:
            oracle.attention_backward(q, inp["k"][ka:ka + n], inp["v"][ka:ka + n], inp["q_gain"], inp["k_gain"],
                                      cfg.eps, cfg.scale, sub, g)
            pairs = n * n
        else:
            sub_text = TextLayout((text.begin[c],), (text.end[c],), text.t_text)
            oracle.cross_attention_backward(q, inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], cfg.eps, cfg.scale,
                                            sub.q_offsets, sub_text, g)
            pairs = n * (text.end[c] - text.begin[c])
        spent = time.perf_counter() - t0
        flops = 2.5 * 4.0 * d * hq * pairs
        if spent > budget_s / 4 or n >= b - a or (text is None and n >= lay.kv_offsets[c + 1] - ka):
            break
        n *= 2
    what = "its text" if text is not None else "itself"
    return {"value": flops / spent / 1e12, "unit": "TFLOP/s", "cores": int(threads), "cpu_model": cpu_model(),
            "kind": "oracle",
            "sample": f"backward of the first {n} tokens of chunk {c} of {cfg.name} attending to {what}, "
                      f"{hq} heads, {spent:.1f} s fp64 numpy on the host"}


def bench_backward(args) -> None:
    """One step = one backward call of the self-attention, or with
    --attention cross of the text cross-attention (the forward's out and lse
    computed once before timing). Useful FLOPs: 2.5 x the forward's (the
    five products S, dP, dV, dK, dQ over the mask area)."""
    import numpy as np
    import torch
    from block_causal_attention_flash_amd import CrossTrainPlan, TrainPlan
    from workloads import get_config, make_inputs, make_text_inputs, text_layout

    cfg = get_config(args.workload)
    if args.kv_range or args.last_global:
        cfg = dataclasses.replace(cfg, layout=dataclasses.replace(cfg.layout, kv_range=args.kv_range,
                                                                  last_global=int(args.last_global)))
    own_dim = args.head_dim in (0, cfg.head_dim)
    if not own_dim:
        cfg = dataclasses.replace(cfg, head_dim=args.head_dim)
    if args.heads:
        hq, hk = (int(x) for x in args.heads.split("/"))
        own_dim = own_dim and (hq, hk) == (cfg.n_q_heads, cfg.n_kv_heads)
        cfg = dataclasses.replace(cfg, n_q_heads=hq, n_kv_heads=hk)
    lay = cfg.layout
    cross = args.attention == "cross"
    dev = torch.device("cuda", 0)
    inp = make_inputs(lay, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype, cfg.gain_kind, cfg.seed)
    text = text_layout(cfg) if cross else None
    if cross:       # the text's keys, values and gains take the places of the video's
        tx = make_text_inputs(text, cfg.n_kv_heads, cfg.head_dim, cfg.dtype, cfg.gain_kind, cfg.seed + 100)
        inp.update(k=tx["k_x"], v=tx["v_x"], q_gain=tx["q_gain_x"], k_gain=tx["k_gain_x"])
    inp["q_gain"] = inp["q_gain"] * args.gain_scale
    g = {n: t.to(dev) for n, t in inp.items()}
    tdt = g["q"].dtype
    dout = torch.from_numpy(np.random.default_rng(cfg.seed + 7).standard_normal(
        (lay.t_q, cfg.n_q_heads, cfg.head_dim), dtype=np.float32)).to(tdt).to(dev)
    t0 = time.perf_counter()
    if cross:
        plan = CrossTrainPlan.from_layout(lay, text, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    else:
        plan = TrainPlan.from_layout(lay, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
    plan_ms = (time.perf_counter() - t0) * 1e3
    stream = torch.cuda.current_stream(dev)
    out, lse = plan(g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], cfg.eps, cfg.scale, stream=stream)
    ws = torch.empty(max(plan.bwd_workspace_size(), 16), dtype=torch.uint8, device=dev)
    dq, dk, dv = torch.empty_like(g["q"]), torch.empty_like(g["k"]), torch.empty_like(g["v"])
    dgq = torch.empty(cfg.head_dim, dtype=torch.float32, device=dev)
    dgk = torch.empty_like(dgq)
    step = lambda: plan.backward(g["q"], g["k"], g["v"], out, lse, dout, g["q_gain"], g["k_gain"], cfg.eps,  # noqa
                                 cfg.scale, dq, dk, dv, dgq, dgk, ws, stream)
    print(f"[bench] {cfg.name} {args.attention} backward: T_q={lay.t_q} "
          f"T_k={text.t_text if cross else lay.t_k} workspace={ws.numel() / 2**30:.2f} GiB "
          f"plan={plan_ms:.1f}ms", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    times, span = step_times(step, stream, args.steps)
    ms = span / args.steps
    pairs = useful_text_pairs(lay, text) if cross else useful_pairs(lay)
    flops = 2.5 * 4.0 * cfg.head_dim * cfg.n_q_heads * pairs
    tflops = flops / (ms * 1e-3) / 1e12
    # The roofline of the whole call (pre-passes, dq, dk/dv, reductions):
    # useful FLOPs over the call's time; traffic is summed over its kernels.
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4),
            "traffic": stored_backward_traffic(cfg.name)
            if cfg.dtype == "bf16" and own_dim
            and not (cross or lay.kv_range or lay.last_global or args.gain_scale != 1.0) else None}
    rec = {
        "metric": METRIC_CROSS_BACKWARD if cross else METRIC_BACKWARD, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": cfg.dtype, "data": "synthetic (seeded N(0,1) Q/K/V/dO)",
        "config": {"workload": cfg.name, "pass": "backward", "attention": args.attention, "t_q": lay.t_q,
                   "t_k": text.t_text if cross else lay.t_k,
                   "n_chunks": lay.n_chunks, "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
                   "head_dim": cfg.head_dim, "kv_range": lay.kv_range, "last_global": lay.last_global,
                   "useful_flops": flops, "unmasked_pairs_per_head": pairs,
                   **({"gain_scale": args.gain_scale} if args.gain_scale != 1.0 else {})},
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4), "plan_create_ms": round(plan_ms, 2),
        "timing": timing_record(times, span, args.steps),
        "roofline": roof, "cpu_baseline": None,
    }
    plan.close()
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU backward oracle on a sample (~{args.cpu_budget / 4:.0f} s)", file=sys.stderr,
              flush=True)
        dout_cpu = dout.cpu()
        host = {n: t for n, t in inp.items()}
        rec["cpu_baseline"] = cpu_baseline_backward(cfg, host, dout_cpu, args.cpu_budget, text)
    print(json.dumps(rec), flush=True)


def copy_probe(mib: int) -> None:
    """A plain copy kernel of known size: reads and writes mib MiB per launch.
    Under rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE its readings give the factor
    between those counters and true HBM bytes."""
    import torch
    n = mib << 20
    src = torch.empty(n, dtype=torch.uint8, device="cuda")
    src.fill_(1)
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_probe_bytes": n, "launches": 3}), flush=True)


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=10)
    ap.add_argument("--warmup", type=int, default=3)
    ap.add_argument("--workload", default="video480x832")
    ap.add_argument("--kv-range", type=int, default=0,
                    help="KV-range window in chunks (0: every earlier chunk of the video is visible)")
    ap.add_argument("--last-global", action="store_true",
                    help="the workload's last video is a global block whose queries see every key of the stream")
    ap.add_argument("--attention", choices=("self", "cross", "parallel"), default="self",
                    help="self: the block-causal self-attention; cross: the text cross-attention of the workload's "
                         "chunk-wise prompts; parallel: both in one launch")
    ap.add_argument("--backward", action="store_true",
                    help="time the backward (magi_attn_bwd) of the self- or (--attention cross) the "
                         "cross-attention instead of the forward")
    ap.add_argument("--gain-scale", type=float, default=1.0,
                    help="multiply the query gains by this factor (larger logits: the static softmax runs with a "
                         "larger shift; work items whose row sums it loses go to the running-maximum instance)")
    ap.add_argument("--cold", action="store_true",
                    help="overwrite a 1 GiB buffer before every timed step (forward), so each step starts with the "
                         "L2s and the Infinity Cache holding other data")
    ap.add_argument("--head-dim", type=int, default=0, choices=(0, 64, 128),
                    help="run the workload at this head_dim instead of its own (64 or 128; the scale follows "
                         "as 1/sqrt(head_dim))")
    ap.add_argument("--heads", default="",
                    help="HQ/HK: run the workload with these head counts instead of its own, e.g. 6/1 for one GPU's "
                         "share of the 48/8 heads sharded by KV head over 8 GPUs")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-budget", type=float, default=20.0)
    ap.add_argument("--copy-probe-mib", type=int, default=0,
                    help="only run a plain device-to-device copy of this many MiB three times (counter calibration)")
    args = ap.parse_args()
    if args.copy_probe_mib:
        copy_probe(args.copy_probe_mib)
        return
    if args.gpus != 1:
        print(f"bench.py measures one GPU; --gpus {args.gpus} is not supported (the kernel runs on one GPU's "
              "share of the work)", file=sys.stderr)
        sys.exit(2)

    if args.backward:
        if args.attention == "parallel":
            print("--backward takes --attention self or cross (the parallel block's backward is the two "
                  "backwards, one per training plan)", file=sys.stderr)
            sys.exit(2)
        return bench_backward(args)
    import torch
    from block_causal_attention_flash_amd import CrossPlan, ParallelPlan, Plan
    from workloads import get_config, make_inputs, make_text_inputs, text_layout

    cfg = get_config(args.workload)
    if args.kv_range or args.last_global:
        cfg = dataclasses.replace(cfg, layout=dataclasses.replace(cfg.layout, kv_range=args.kv_range,
                                                                  last_global=int(args.last_global)))
    own_dim = args.head_dim in (0, cfg.head_dim)
    if not own_dim:
        cfg = dataclasses.replace(cfg, head_dim=args.head_dim)
    if args.heads:
        hq, hk = (int(x) for x in args.heads.split("/"))
        own_dim = own_dim and (hq, hk) == (cfg.n_q_heads, cfg.n_kv_heads)
        cfg = dataclasses.replace(cfg, n_q_heads=hq, n_kv_heads=hk)
    lay = cfg.layout
    mode = args.attention
    text = text_layout(cfg) if mode != "self" else None
    dev = torch.device("cuda", 0)
    t0 = time.perf_counter()
    inp = make_inputs(lay, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype, cfg.gain_kind, cfg.seed)
    tx = (make_text_inputs(text, cfg.n_kv_heads, cfg.head_dim, cfg.dtype, cfg.gain_kind, cfg.seed + 100)
          if text is not None else None)
    if args.gain_scale != 1.0:
        inp["q_gain"] = inp["q_gain"] * args.gain_scale
        if tx is not None:
            tx["q_gain_x"] = tx["q_gain_x"] * args.gain_scale
    gen_s = time.perf_counter() - t0
    g = lambda t: t.to(dev)  # noqa: E731
    q = g(inp["q"])
    lse_shape = (cfg.n_q_heads, lay.t_q)
    out, lse = torch.empty_like(q), torch.empty(lse_shape, dtype=torch.float32, device=dev)
    t0 = time.perf_counter()
    # The workspace is allocated once, as a training or serving loop would.
    if mode == "self":
        plan = Plan.from_layout(lay, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
        ws = torch.empty(max(plan.workspace_size(), 16), dtype=torch.uint8, device=dev)
        k, v, qg, kg = g(inp["k"]), g(inp["v"]), g(inp["q_gain"]), g(inp["k_gain"])
        step = lambda: plan(q, k, v, qg, kg, cfg.eps, cfg.scale, out=out, lse=lse, workspace=ws,  # noqa: E731
                            stream=stream)
    elif mode == "cross":
        plan = CrossPlan.from_layout(lay, text, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
        ws = torch.empty(max(plan.workspace_size(), 16), dtype=torch.uint8, device=dev)
        kx, vx, qgx, kgx = g(tx["k_x"]), g(tx["v_x"]), g(tx["q_gain_x"]), g(tx["k_gain_x"])
        step = lambda: plan(q, kx, vx, qgx, kgx, cfg.eps, cfg.scale, out=out, lse=lse, workspace=ws,  # noqa: E731
                            stream=stream)
    else:
        plan = ParallelPlan.from_layout(lay, text, cfg.n_q_heads, cfg.n_kv_heads, cfg.head_dim, cfg.dtype)
        ws = torch.empty(max(plan.workspace_size(), 16), dtype=torch.uint8, device=dev)
        k, v, qg, kg = g(inp["k"]), g(inp["v"]), g(inp["q_gain"]), g(inp["k_gain"])
        kx, vx, qgx, kgx = g(tx["k_x"]), g(tx["v_x"]), g(tx["q_gain_x"]), g(tx["k_gain_x"])
        out_x, lse_x = torch.empty_like(q), torch.empty(lse_shape, dtype=torch.float32, device=dev)
        step = lambda: plan(q, k, v, kx, vx, q_gain=qg, k_gain=kg, q_gain_x=qgx, k_gain_x=kgx,  # noqa: E731
                            rms_eps=cfg.eps, scale=cfg.scale, scale_x=cfg.scale, out=out, lse=lse, out_x=out_x,
                            lse_x=lse_x, workspace=ws, stream=stream)
    plan_ms = (time.perf_counter() - t0) * 1e3
    stats = plan.stats()
    print(f"[bench] {cfg.name} ({mode}): T_q={lay.t_q} T_k={lay.t_k}"
          f"{'' if text is None else f' T_text={text.t_text}'} heads {cfg.n_q_heads}/{cfg.n_kv_heads} "
          f"items={stats['n_items']} gen={gen_s:.1f}s plan={plan_ms:.1f}ms", file=sys.stderr, flush=True)

    stream = torch.cuda.current_stream(dev)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    # --cold: a buffer larger than the L2s and the 256 MB Infinity Cache is
    # overwritten before every step (outside the timed events)
    flush = torch.empty(1 << 30, dtype=torch.uint8, device=dev) if args.cold else None
    wall0 = time.perf_counter()
    times, span = step_times(step, stream, args.steps, flush)
    wall_ms = (time.perf_counter() - wall0) * 1e3 / args.steps
    ms = span / args.steps
    print(f"[bench] {args.steps} steps{' (cold caches)' if args.cold else ''}: {ms:.3f} ms/step mean, "
          f"median {sorted(times)[len(times) // 2]:.3f}, min {min(times):.3f} (events); {wall_ms:.3f} ms/step host wall",
          file=sys.stderr, flush=True)

    pairs = useful_pairs(lay) if mode != "cross" else 0
    pairs_x = useful_text_pairs(lay, text) if mode != "self" else 0
    flops = 4.0 * cfg.head_dim * cfg.n_q_heads * (pairs + pairs_x)
    tflops = flops / (ms * 1e-3) / 1e12
    # the stored counters belong to the static-softmax instance on the workload's own gains
    traffic = (stored_traffic(cfg.name, mode)
               if own_dim and not (lay.kv_range or lay.last_global or args.gain_scale != 1.0 or args.cold) else None)
    roof = {"bound": "mfma", "achieved": round(tflops, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
            "frac": round(tflops / PEAK_BF16_TFLOPS, 4), "traffic": traffic}
    if traffic:
        roof["hbm_gbps"] = round(traffic / (ms * 1e-3) / 1e9, 1)

    cpu = None
    if not args.no_cpu_baseline:
        print(f"[bench] timing the CPU oracle on a sample (~{args.cpu_budget:.0f} s)", file=sys.stderr, flush=True)
        cpu = cpu_baseline(cfg, inp, args.cpu_budget, mode, text, tx)

    config = {"workload": cfg.name, "attention": mode, "t_q": lay.t_q, "t_k": lay.t_k, "n_chunks": lay.n_chunks,
              "n_videos": lay.n_seqs, "n_q_heads": cfg.n_q_heads, "n_kv_heads": cfg.n_kv_heads,
              "head_dim": cfg.head_dim, "kv_range": lay.kv_range, "last_global": lay.last_global,
              "useful_flops": flops, "unmasked_pairs_per_head": pairs}
    if args.gain_scale != 1.0:
        config["gain_scale"] = args.gain_scale
    if text is not None:
        config.update({"t_text": text.t_text, "text_pairs_per_head": pairs_x})
    if args.cold:
        config["caches"] = "cold (1 GiB written between steps)"
    rec = {
        "metric": METRIC if mode == "self" else METRIC_CROSS if mode == "cross" else METRIC_PARALLEL,
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": cfg.dtype,
        "data": "synthetic (seeded N(0,1) Q/K/V, unit QK-norm gains)" if cfg.gain_kind == "ones" else
                "synthetic (seeded N(0,1) Q/K/V, QK-norm gains U(0.5,1.5))",
        "config": config,
        "frac_of_peak": round(tflops / PEAK_BF16_TFLOPS, 4),
        "plan_create_ms": round(plan_ms, 2),
        "timing": timing_record(times, span, args.steps),
        "roofline": roof,
        "cpu_baseline": cpu,
    }
    plan.close()
    print(json.dumps(rec), flush=True)


if __name__ == "__main__":
    main()
