"""magi_attn_fwd_noalloc (the forward with the library's static device
scratch as its workspace, for callers that cannot allocate) against
magi_attn_fwd with a caller workspace, through the C ABI.

Calls in a row on different plans (head_dim 128 and 64), the last smaller than
the others, so that each reads a scratch array still holding the previous call's images,
partial results and flags: each output must equal magi_attn_fwd's bit for bit
(same kernels, same inputs), and both are checked against the fp64 oracle at
the bf16 tolerances. Outputs start as NaN, so an element the call does not
write fails. A plan whose workspace exceeds the scratch is refused.
"""
import math
import sys

import numpy as np
import pytest
import torch

import oracle
from workloads import Layout, layout_from_chunks, make_inputs

pytestmark = pytest.mark.gpu

DEV = torch.device("cuda", 0)
SC = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module", autouse=True)
def _gpu(built_lib):
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    return built_lib


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def split_layout():
    """A KV cache of 12 chunks of 512 keys read by two 96-token chunks: too few
    work items, so the plan splits them and the call uses the scratch's
    partial-result slots and the merge."""
    kv = [512 * i for i in range(13)] + [6144 + 1024, 6144 + 2048]
    q = [0] * 13 + [96, 192]
    return Layout(tuple(q), tuple(kv), (0, 14))


CASES = [
    ("two videos, 6/2", layout_from_chunks([[300, 157, 91], [200, 64]]), 6, 2, 128, 31),
    ("split KV cache, 8/2", split_layout(), 8, 2, 128, 32),
    ("split KV cache, 8/2, head_dim 64", split_layout(), 8, 2, 64, 34),
    ("one small chunk, 3/1", layout_from_chunks([[130, 70]]), 3, 1, 128, 33),
]


def _run_pair(lay, hq, hk, d, seed):
    from block_causal_attention_flash_amd import Plan, magi_attn_fwd, magi_attn_fwd_noalloc, magi_attn_plan_stats
    sc = 1.0 / math.sqrt(d)
    inp = make_inputs(lay, hq, hk, d, "bf16", "uniform", seed)
    g = {n: t.to(DEV) for n, t in inp.items()}
    plan = Plan.from_layout(lay, hq, hk, d, "bf16")
    st = magi_attn_plan_stats(lay.q_offsets, lay.kv_offsets, lay.seq_chunks, hq, hk, d, "bf16")
    out_a = torch.full_like(g["q"], float("nan"))
    lse_a = torch.full((hq, lay.t_q), float("nan"), dtype=torch.float32, device=DEV)
    ws = torch.empty(max(plan.workspace_size(), 16), dtype=torch.uint8, device=DEV)
    magi_attn_fwd(plan.handle, g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], 1e-6, sc, out=out_a, lse=lse_a,
                  workspace=ws)
    out_b = torch.full_like(g["q"], float("nan"))
    lse_b = torch.full((hq, lay.t_q), float("nan"), dtype=torch.float32, device=DEV)
    magi_attn_fwd_noalloc(plan.handle, g["q"], g["k"], g["v"], g["q_gain"], g["k_gain"], 1e-6, sc, out_b, lse_b)
    torch.cuda.synchronize()
    assert torch.equal(out_a, out_b) and torch.equal(lse_a, lse_b)
    ro, rl = oracle.attention(inp["q"], inp["k"], inp["v"], inp["q_gain"], inp["k_gain"], 1e-6, sc, lay)
    got = out_b.double().cpu().numpy()
    gl = lse_b.double().cpu().numpy()
    rl2 = float(np.linalg.norm(got - ro) / np.linalg.norm(ro))
    mabs = float(np.max(np.abs(got - ro)))
    lerr = float(np.max(np.abs(gl - rl)))
    assert rl2 <= 5e-3 and mabs <= 2e-2 and lerr <= 1e-2, (rl2, mabs, lerr)
    ws_bytes = plan.workspace_size()
    plan.close()
    return ws_bytes, st["n_items"], rl2


def test_noalloc_equals_fwd_on_consecutive_calls():
    sizes = []
    for name, lay, hq, hk, d, seed in CASES:
        log(f"noalloc: {name}")
        ws_bytes, n_items, rl2 = _run_pair(lay, hq, hk, d, seed)
        log(f"noalloc: {name}: workspace {ws_bytes} bytes, {n_items} items, rel_l2 {rl2:.3e}")
        sizes.append(ws_bytes)
    assert all(sizes[-1] < x for x in sizes[:-1])         # the last call is the smallest


def test_noalloc_refuses_a_workspace_beyond_the_scratch():
    from block_causal_attention_flash_amd import MagiAttnError, Plan, magi_attn_fwd_noalloc
    from block_causal_attention_flash_amd._abi import MAGI_ATTN_NOALLOC_SCRATCH_BYTES
    lay = Layout((0, 0, 64), (0, 70000, 70064), (0, 2))   # 8 KV heads x 70,064 keys: 287 MB of tile images
    plan = Plan.from_layout(lay, 8, 8, 128, "bf16")
    assert plan.workspace_size() > MAGI_ATTN_NOALLOC_SCRATCH_BYTES
    q = torch.zeros((64, 8, 128), dtype=torch.bfloat16, device=DEV)
    kv = torch.zeros((70064, 8, 128), dtype=torch.bfloat16, device=DEV)
    gains = torch.ones(128, dtype=torch.float32, device=DEV)
    out = torch.empty_like(q)
    lse = torch.empty((8, 64), dtype=torch.float32, device=DEV)
    with pytest.raises(MagiAttnError) as e:
        magi_attn_fwd_noalloc(plan.handle, q, kv, kv, gains, gains, 1e-6, SC, out, lse)
    assert e.value.status == 2 and "static scratch" in e.value.message
    plan.close()
