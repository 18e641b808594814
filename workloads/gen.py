"""Seeded input tensors: Q, K, V ~ N(0, 1) and the QK-norm gains.

Values are drawn in float32 with numpy's default_rng(seed) and, for bf16
workloads, rounded once to bfloat16 (round-to-nearest-even, by torch on the
CPU). The same rounded tensors go to the GPU and, upcast losslessly to float64,
to the oracle.
"""
from __future__ import annotations

from typing import Dict, Optional

import numpy as np
import torch


def _normal(rng, shape):
    return rng.standard_normal(shape, dtype=np.float32)


def make_inputs(layout, n_q_heads: int, n_kv_heads: int, head_dim: int, dtype: str = "bf16",
                gain_kind: str = "ones", seed: int = 0) -> Dict[str, torch.Tensor]:
    """Returns CPU tensors q [T_q,H_q,d], k/v [T_k,H_k,d] in `dtype`, and fp32
    gains q_gain/k_gain [d]."""
    rng = np.random.default_rng(seed)
    tq, tk = int(layout.q_offsets[-1]), int(layout.kv_offsets[-1])
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    q = torch.from_numpy(_normal(rng, (tq, n_q_heads, head_dim))).to(tdt)
    k = torch.from_numpy(_normal(rng, (tk, n_kv_heads, head_dim))).to(tdt)
    v = torch.from_numpy(_normal(rng, (tk, n_kv_heads, head_dim))).to(tdt)
    if gain_kind == "ones":
        qg = np.ones(head_dim, np.float32)
        kg = np.ones(head_dim, np.float32)
    elif gain_kind == "uniform":
        qg = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
        kg = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
    else:
        raise ValueError(gain_kind)
    return {"q": q, "k": k, "v": v, "q_gain": torch.from_numpy(qg), "k_gain": torch.from_numpy(kg)}


def make_text_inputs(text, n_kv_heads: int, head_dim: int, dtype: str = "bf16", gain_kind: str = "ones",
                     seed: int = 0) -> Dict[str, torch.Tensor]:
    """Text keys/values k_x, v_x [T_text,H_k,d] ~ N(0,1) in `dtype` and the
    cross-attention's own QK-norm gains q_gain_x / k_gain_x [d] (fp32), drawn
    with default_rng(seed) in that order."""
    rng = np.random.default_rng(seed)
    tdt = {"bf16": torch.bfloat16, "fp32": torch.float32}[dtype]
    k = torch.from_numpy(_normal(rng, (int(text.t_text), n_kv_heads, head_dim))).to(tdt)
    v = torch.from_numpy(_normal(rng, (int(text.t_text), n_kv_heads, head_dim))).to(tdt)
    if gain_kind == "ones":
        qg = np.ones(head_dim, np.float32)
        kg = np.ones(head_dim, np.float32)
    elif gain_kind == "uniform":
        qg = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
        kg = rng.uniform(0.5, 1.5, head_dim).astype(np.float32)
    else:
        raise ValueError(gain_kind)
    return {"k_x": k, "v_x": v, "q_gain_x": torch.from_numpy(qg), "k_gain_x": torch.from_numpy(kg)}
