"""fp64 CPU oracle of the text cross-attention of MAGI-1's parallel attention block.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library.

What is computed (MAGI-1 pages):
  * paperlayer summary §2.2.2 and paper-notes §3.2.2 (architecture list,
    Figure 3 reading, DiT-block pseudocode): every transformer block runs the
    spatial-temporal self-attention and a cross-attention to the text
    condition side by side, both from one shared query projection; QK-Norm and
    grouped-query attention apply to the cross-attention too, with the same
    head layout (the paper-notes spec table lists "Cross Attn Heads" with
    8 groups, as for self-attention);
  * paperlayer §2.2.3: prompts are given per chunk ("chunk-wise prompts"),
    so different chunks of one video may attend to different text;
  * paper-notes §3.2.6 (clean chunks): chunks that are already clean carry no
    text condition.

Readings taken where the pages are silent or garbled:
  * chunk c's queries attend, without any mask, to the text tokens
    [text.begin[c], text.end[c]) of one packed text stream; a chunk with
    begin == end has no text (a clean chunk);
  * a query row with no key at all has out = 0 and lse = -inf (the empty sum:
    such a row adds nothing to the block's output, and a partial result with
    lse = -inf carries zero weight in the log-sum-exp merge);
  * q and the text keys are RMS-normalised over head_dim with their own gains;
    the values are not normalised (the paper-notes pseudocode also normalises
    v_cross and leaves q un-normalised there, which contradicts the notes' own
    statement that QK-Norm applies to the cross-attention: taken as a slip);
  * the cross branch uses the query projection without RoPE (text tokens have
    no video position), so its q may differ from the self-attention's q.

Every function below is the plain definition, written out without tiling.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np

from . import dense


def text_mask(q_offsets: Sequence[int], text, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Dense boolean mask M[i, j] over (query row, text key): true when key j
    lies in the text range of query i's chunk."""
    tq = int(q_offsets[-1])
    qc = dense.token_chunk_ids(q_offsets, tq)
    if rows is not None:
        qc = qc[np.asarray(rows)]
    begin = np.asarray(text.begin, dtype=np.int64)
    end = np.asarray(text.end, dtype=np.int64)
    j = np.arange(int(text.t_text), dtype=np.int64)
    return (j[None, :] >= begin[qc][:, None]) & (j[None, :] < end[qc][:, None])


def text_pairs(q_offsets: Sequence[int], text) -> int:
    """Allowed (query, text key) pairs per query head: the FLOP area of the
    cross-attention (paperlayer §B.2.1 accounting, as for self-attention)."""
    return int(sum((q_offsets[c + 1] - q_offsets[c]) * (text.end[c] - text.begin[c])
                   for c in range(len(q_offsets) - 1)))


def cross_attention(q, k, v, q_gain, k_gain, eps: float, scale: float, q_offsets: Sequence[int], text,
                    rows: Optional[Sequence[int]] = None, row_block: int = 256) -> Tuple[np.ndarray, np.ndarray]:
    """Softmax attention of the video queries over the text keys, in float64.

    q: [T_q, H_q, d]; k, v: [T_text, H_kv, d]; gains: [d]. Query head h uses
    text KV head h // (H_q / H_kv). Returns out [R, H_q, d] and lse [H_q, R]
    (natural log), R = len(rows); rows without text: out 0, lse -inf.
    """
    q = dense._as_f64(q)
    k = dense._as_f64(k)
    v = dense._as_f64(v)
    tq, hq, d = q.shape
    hk = k.shape[1]
    if hq % hk != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    group = hq // hk
    rows = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    qh = dense.rms_norm(q[rows], q_gain, eps)
    kh = dense.rms_norm(k, k_gain, eps)
    out = np.zeros((len(rows), hq, d), dtype=np.float64)
    lse = np.full((hq, len(rows)), -np.inf, dtype=np.float64)
    for r0 in range(0, len(rows), row_block):
        sel = np.arange(r0, min(len(rows), r0 + row_block))
        mask = text_mask(q_offsets, text, rows[sel])
        live = mask.any(axis=1)
        if not live.any():
            continue
        sel, mask = sel[live], mask[live]
        for h in range(hq):
            g = h // group
            s = scale * (qh[sel, h, :] @ kh[:, g, :].T)
            s = np.where(mask, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            p = np.exp(s - m)
            l = np.sum(p, axis=1, keepdims=True)
            out[sel, h, :] = (p @ v[:, g, :]) / l
            lse[h, sel] = (m + np.log(l))[:, 0]
    return out, lse


def cross_attention_loops(q, k, v, q_gain, k_gain, eps: float, scale: float, q_offsets: Sequence[int], text
                          ) -> Tuple[np.ndarray, np.ndarray]:
    """Brute force with pure-Python loops, math.exp and math.fsum: a text key
    j is allowed for query i when begin[c] <= j < end[c], c = chunk of i.
    Independent of text_mask and of numpy's reductions. Tiny inputs only."""
    q = dense._as_f64(q).tolist()
    k = dense._as_f64(k).tolist()
    v = dense._as_f64(v).tolist()
    qg = [float(x) for x in dense._as_f64(q_gain)]
    kg = [float(x) for x in dense._as_f64(k_gain)]
    tq = len(q)
    hq, hk, d = len(q[0]), len(k[0]), len(q[0][0])
    group = hq // hk

    def norm(vec, gain):
        inv = 1.0 / math.sqrt(math.fsum(x * x for x in vec) / len(vec) + eps)
        return [x * g * inv for x, g in zip(vec, gain)]

    out = [[[0.0] * d for _ in range(hq)] for _ in range(tq)]
    lse = [[-math.inf] * tq for _ in range(hq)]
    for i in range(tq):
        c = next(c for c in range(len(q_offsets) - 1) if q_offsets[c] <= i < q_offsets[c + 1])
        keys = list(range(int(text.begin[c]), int(text.end[c])))
        if not keys:
            continue
        for h in range(hq):
            g = h // group
            qi = norm(q[i][h], qg)
            scores = [scale * math.fsum(a * b for a, b in zip(qi, norm(k[j][g], kg))) for j in keys]
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            l = math.fsum(w)
            for e in range(d):
                out[i][h][e] = math.fsum(wj * v[j][g][e] for wj, j in zip(w, keys)) / l
            lse[h][i] = m + math.log(l)
    return np.array(out), np.array(lse)
