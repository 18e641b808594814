"""fp64 CPU oracle of block-causal, QK-RMS-normalised, grouped-query attention.

TEST INFRASTRUCTURE ONLY. Nothing on the product path may import, call or
execute this module: only the tests, the smoke check and the benchmark's CPU
baseline leg use it. It shares no code with the HIP library.

What is computed (MAGI-1 pages):
  * paperlayer summary §2 and Figure 1, paper-notes §2 and its Figure 1 reading:
    attention is bidirectional among the tokens of one chunk and causal across
    chunks; a chunk sees itself and every earlier chunk of the same video.
  * paper-notes Figure 15 (AttnSlice mask catalogue, "varlen block-causal"):
    videos packed into one stream never attend to each other.
  * paperlayer §2.2.2 and paper-notes §3.2.2 (architecture bullets, the DiT
    block pseudocode): queries and keys are normalised per head before the
    product ("QK-Norm"), and several query heads share one key/value head
    (GQA, 8 KV groups in the paper-notes spec table).
  * paperlayer §2.4.4: keys/values of clean chunks come from a KV cache, so the
    key stream may be longer than the query stream.

Readings taken where the pages are silent or garbled:
  * the QK normalisation is RMSNorm over head_dim with a per-channel gain g
    shared by all heads:  x_hat = x * g / sqrt(mean_d(x^2) + eps);
  * query head h uses key/value head h // (H_q / H_kv) (contiguous groups);
  * s_ij = scale * <q_hat_i, k_hat_j>, masked entries are -inf, softmax over j;
  * the log-sum-exp is natural-log: lse_i = m_i + ln(sum_j exp(s_ij - m_i)).

Every function below is the plain definition, written out without tiling.
"""
from __future__ import annotations

import math
from typing import Optional, Sequence, Tuple

import numpy as np


def _as_f64(x) -> np.ndarray:
    """Lossless upcast of a numpy array or a (CPU) torch tensor to float64."""
    if hasattr(x, "detach"):
        x = x.detach().to("cpu")
        import torch
        x = x.to(torch.float64).numpy()
    return np.asarray(x, dtype=np.float64)


def rms_norm(x, gain, eps: float) -> np.ndarray:
    """RMSNorm over the last axis (head_dim) with a per-channel gain.

    paper-notes §3.2.2 places the QK-Norm right before the block-causal
    attention call; the RMS form with gain is the reading taken (an L2 norm
    differs from it only by the constant sqrt(d), which would move into the
    temperature).
    """
    x = _as_f64(x)
    g = _as_f64(gain)
    ms = np.mean(x * x, axis=-1, keepdims=True)
    return x * g / np.sqrt(ms + eps)


def token_chunk_ids(offsets: Sequence[int], total: int) -> np.ndarray:
    """Chunk index of every token of a packed stream: token t belongs to chunk c
    when offsets[c] <= t < offsets[c+1]."""
    offsets = np.asarray(offsets, dtype=np.int64)
    ids = np.full(total, -1, dtype=np.int64)
    for c in range(len(offsets) - 1):
        ids[offsets[c]:offsets[c + 1]] = c
    return ids


def chunk_video_ids(seq_chunks: Sequence[int], n_chunks: int) -> np.ndarray:
    """Video index of every chunk: chunk c belongs to video s when
    seq_chunks[s] <= c < seq_chunks[s+1]."""
    ids = np.full(n_chunks, -1, dtype=np.int64)
    for s in range(len(seq_chunks) - 1):
        ids[seq_chunks[s]:seq_chunks[s + 1]] = s
    return ids


def block_causal_mask(layout, rows: Optional[np.ndarray] = None) -> np.ndarray:
    """Dense boolean mask M[i, j] over (query row, key) of the packed streams.

    M[i, j] is true when key j lies in the same video as query i and its chunk
    is not later than the query's chunk (paperlayer §2 / Figure 1: bidirectional
    within a chunk, causal across chunks; paper-notes Figure 15: no attention
    across packed videos). With a KV range R >= 1 (layout.kv_range; paperlayer
    §2.4.4, paper-notes §3.4.4 and Figure 12) the key's chunk must also be one
    of the query chunk's R latest: kc > qc - R. With layout.last_global set, the
    last video of the stream is a global block (paper-notes Figure 15(g),
    paperlayer Figure 23: varlen block-causal with a last global block): its
    queries see every key of the stream.
    """
    tq, tk = int(layout.q_offsets[-1]), int(layout.kv_offsets[-1])
    n_chunks = len(layout.q_offsets) - 1
    qc = token_chunk_ids(layout.q_offsets, tq)
    kc = token_chunk_ids(layout.kv_offsets, tk)
    vid = chunk_video_ids(layout.seq_chunks, n_chunks)
    if rows is not None:
        qc = qc[np.asarray(rows)]
    same_video = vid[qc][:, None] == vid[kc][None, :]
    not_later = kc[None, :] <= qc[:, None]
    mask = same_video & not_later
    R = int(getattr(layout, "kv_range", 0))
    if R > 0:
        mask &= kc[None, :] > qc[:, None] - R
    if int(getattr(layout, "last_global", 0)):
        mask[vid[qc] == n_seqs_of(layout) - 1, :] = True
    return mask


def n_seqs_of(layout) -> int:
    return len(layout.seq_chunks) - 1


def unmasked_pairs(layout) -> int:
    """Number of allowed (query, key) pairs per query head: the mask area that
    the forward FLOP count is taken over (paperlayer §B.2.1: two matmuls over
    the mask area, following Flash-Attention)."""
    tq = int(layout.q_offsets[-1])
    total = 0
    for r0 in range(0, tq, 2048):
        total += int(block_causal_mask(layout, np.arange(r0, min(tq, r0 + 2048))).sum())
    return total


def attention(q, k, v, q_gain, k_gain, eps: float, scale: float, layout,
              rows: Optional[Sequence[int]] = None, row_block: int = 256
              ) -> Tuple[np.ndarray, np.ndarray]:
    """Masked softmax attention in float64.

    q: [T_q, H_q, d]; k, v: [T_k, H_kv, d]; gains: [d].
    rows: optional subset of query rows (token indices); default all.
    Returns out [R, H_q, d] and lse [H_q, R] (natural log), R = len(rows).
    """
    q = _as_f64(q)
    k = _as_f64(k)
    v = _as_f64(v)
    tq, hq, d = q.shape
    tk, hk, _ = k.shape
    if hq % hk != 0:
        raise ValueError("n_q_heads must be a multiple of n_kv_heads")
    group = hq // hk
    rows = np.arange(tq) if rows is None else np.asarray(rows, dtype=np.int64)
    qh = rms_norm(q[rows], q_gain, eps)          # [R, H_q, d]
    kh = rms_norm(k, k_gain, eps)                # [T_k, H_kv, d]
    out = np.zeros((len(rows), hq, d), dtype=np.float64)
    lse = np.zeros((hq, len(rows)), dtype=np.float64)
    for r0 in range(0, len(rows), row_block):
        sel = slice(r0, min(len(rows), r0 + row_block))
        mask = block_causal_mask(layout, rows[sel])          # [b, T_k]
        for h in range(hq):
            g = h // group
            s = scale * (qh[sel, h, :] @ kh[:, g, :].T)      # [b, T_k]
            s = np.where(mask, s, -np.inf)
            m = np.max(s, axis=1, keepdims=True)
            p = np.exp(s - m)
            l = np.sum(p, axis=1, keepdims=True)
            out[sel, h, :] = (p @ v[:, g, :]) / l
            lse[h, sel] = (m + np.log(l))[:, 0]
    return out, lse


def attention_probs(q, k, q_gain, k_gain, eps: float, scale: float, layout) -> np.ndarray:
    """The full softmax matrix P [H_q, T_q, T_k] (small inputs only)."""
    q = _as_f64(q)
    k = _as_f64(k)
    tq, hq, d = q.shape
    hk = k.shape[1]
    group = hq // hk
    qh = rms_norm(q, q_gain, eps)
    kh = rms_norm(k, k_gain, eps)
    mask = block_causal_mask(layout)
    probs = np.zeros((hq, tq, k.shape[0]), dtype=np.float64)
    for h in range(hq):
        s = scale * (qh[:, h, :] @ kh[:, h // group, :].T)
        s = np.where(mask, s, -np.inf)
        p = np.exp(s - np.max(s, axis=1, keepdims=True))
        probs[h] = p / np.sum(p, axis=1, keepdims=True)
    return probs


def attention_loops(q, k, v, q_gain, k_gain, eps: float, scale: float, layout
                    ) -> Tuple[np.ndarray, np.ndarray]:
    """Brute force with pure-Python per-token loops, math.exp and math.fsum.

    Independent of numpy's reductions and of the dense-mask construction: a
    key is allowed for a query when both chunks belong to the same video and
    the key's chunk index is not larger than the query's (and, with a KV range
    R, larger than the query's minus R); a query of a last global block sees
    every key. Tiny inputs only.
    """
    q = _as_f64(q).tolist()
    k = _as_f64(k).tolist()
    v = _as_f64(v).tolist()
    qg = [float(x) for x in _as_f64(q_gain)]
    kg = [float(x) for x in _as_f64(k_gain)]
    tq, tk = len(q), len(k)
    hq, hk, d = len(q[0]), len(k[0]), len(q[0][0])
    group = hq // hk

    def chunk_of(offsets, t):
        for c in range(len(offsets) - 1):
            if offsets[c] <= t < offsets[c + 1]:
                return c
        raise ValueError("token outside layout")

    def video_of(c):
        for s in range(len(layout.seq_chunks) - 1):
            if layout.seq_chunks[s] <= c < layout.seq_chunks[s + 1]:
                return s
        raise ValueError("chunk outside layout")

    def norm(vec, gain):
        ms = math.fsum(x * x for x in vec) / len(vec)
        inv = 1.0 / math.sqrt(ms + eps)
        return [x * g * inv for x, g in zip(vec, gain)]

    out = [[[0.0] * d for _ in range(hq)] for _ in range(tq)]
    lse = [[0.0] * tq for _ in range(hq)]
    kchunks = [chunk_of(layout.kv_offsets, j) for j in range(tk)]
    for i in range(tq):
        ci = chunk_of(layout.q_offsets, i)
        R = int(getattr(layout, "kv_range", 0))
        if int(getattr(layout, "last_global", 0)) and video_of(ci) == len(layout.seq_chunks) - 2:
            allowed = list(range(tk))             # a query of the global block sees every key
        else:
            allowed = [j for j in range(tk)
                       if video_of(kchunks[j]) == video_of(ci) and kchunks[j] <= ci and (R == 0 or kchunks[j] > ci - R)]
        for h in range(hq):
            g = h // group
            qi = norm(q[i][h], qg)
            scores = [scale * math.fsum(a * b for a, b in zip(qi, norm(k[j][g], kg))) for j in allowed]
            m = max(scores)
            w = [math.exp(s - m) for s in scores]
            l = math.fsum(w)
            for c in range(d):
                out[i][h][c] = math.fsum(wj * v[j][g][c] for wj, j in zip(w, allowed)) / l
            lse[h][i] = m + math.log(l)
    return np.array(out), np.array(lse)
