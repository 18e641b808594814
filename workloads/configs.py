"""Chunk layouts of the benchmark workloads (pure bookkeeping, no attention math).

A layout describes a packed token stream the way the block-causal problem is
stated on the MAGI-1 pages (paperlayer summary §2 and Figure 1; paper-notes
§2 and Figure 1): a video is a sequence of 24-frame chunks, several videos may
be packed into one stream (paper-notes Figure 15, "varlen block-causal"), and
the keys of already-denoised chunks may come from a KV cache (paperlayer §2.4.4).

Fields (all offsets are token indices into the packed streams):
  q_offsets[n_chunks+1]   chunk c owns queries  [q_offsets[c],  q_offsets[c+1])
  kv_offsets[n_chunks+1]  chunk c owns keys     [kv_offsets[c], kv_offsets[c+1])
  seq_chunks[n_seqs+1]    video s owns chunks   [seq_chunks[s], seq_chunks[s+1])

Token counts follow the pages' VAE compression (8x spatial, 4x temporal,
paperlayer §2.1): a 24-frame chunk is 6 latent frames, and with a 2x2 patch a
latent frame of H/8 x W/8 becomes (H/16)*(W/16) tokens.
"""
from __future__ import annotations

import dataclasses
import math
from typing import List, Optional, Sequence

import numpy as np


@dataclasses.dataclass(frozen=True)
class Layout:
    q_offsets: tuple
    kv_offsets: tuple
    seq_chunks: tuple
    kv_range: int = 0      # 0: block-causal; R >= 1: a chunk sees the last R chunks of its video
    last_global: int = 0   # 1: the last video is a global block whose queries see every key of the stream

    @property
    def n_chunks(self) -> int:
        return len(self.q_offsets) - 1

    @property
    def n_seqs(self) -> int:
        return len(self.seq_chunks) - 1

    @property
    def t_q(self) -> int:
        return int(self.q_offsets[-1])

    @property
    def t_k(self) -> int:
        return int(self.kv_offsets[-1])


def layout_from_chunks(videos: Sequence[Sequence[int]]) -> Layout:
    """Self-attention layout: each video is a list of chunk token counts; the
    query and key streams are the same packed stream."""
    offs = [0]
    seq = [0]
    for vid in videos:
        for n in vid:
            offs.append(offs[-1] + int(n))
        seq.append(len(offs) - 1)
    return Layout(tuple(offs), tuple(offs), tuple(seq))


def streaming_layout(n_cached: int, n_active: int, chunk_tokens: int) -> Layout:
    """One video whose first n_cached chunks are clean (keys/values only, read
    from the KV cache) and whose last n_active chunks are being denoised
    (queries and keys/values)."""
    n = n_cached + n_active
    q = [max(0, c - n_cached) * chunk_tokens for c in range(n + 1)]
    kv = [c * chunk_tokens for c in range(n + 1)]
    return Layout(tuple(q), tuple(kv), (0, n))


def packed_chunk_draw(seed: int = 8):
    """The packed-batch draw: 8 videos, each with 1..10 chunks of one size from
    {256, 1536, 3840, 9360}; seed 8 is the first seed whose total lies within
    2% of 120k tokens (121,152)."""
    sizes = np.array([256, 1536, 3840, 9360])
    rng = np.random.default_rng(seed)
    n = rng.integers(1, 11, 8)
    sz = sizes[rng.integers(0, 4, 8)]
    return [[int(s)] * int(c) for c, s in zip(n, sz)]


@dataclasses.dataclass(frozen=True)
class TextLayout:
    """Text side of the cross-attention: chunk c's queries attend to the text
    keys [begin[c], end[c]) of one packed text stream of t_text tokens;
    begin[c] == end[c] means the chunk has no text condition (a clean chunk).
    Chunk-wise prompts: paperlayer §2.2.3; clean chunks without text:
    paper-notes §3.2.6."""
    begin: tuple
    end: tuple
    t_text: int


def chunk_prompts(prompt_of_chunk: Sequence[Optional[int]], prompt_lengths: Sequence[int]) -> TextLayout:
    """Prompts packed one after another into the text stream; chunk c uses
    prompt prompt_of_chunk[c], or no text when that entry is None."""
    starts = [0]
    for n in prompt_lengths:
        starts.append(starts[-1] + int(n))
    begin = tuple(0 if p is None else starts[p] for p in prompt_of_chunk)
    end = tuple(0 if p is None else starts[p + 1] for p in prompt_of_chunk)
    return TextLayout(begin, end, starts[-1])


def prompt_draw(layout: Layout, clean_per_video: int, chunks_per_prompt: int, seed: int, lo: int = 64,
                hi: int = 512) -> TextLayout:
    """Chunk-wise prompts for a layout: in every video the first
    `clean_per_video` chunks carry no text, and each following run of
    `chunks_per_prompt` chunks shares one prompt; chunks without queries (a
    KV cache) carry none either. Prompt lengths are drawn uniformly from
    [lo, hi] tokens with default_rng(seed), in prompt order."""
    prompt_of_chunk: List[Optional[int]] = []
    n_prompts = 0
    for s in range(layout.n_seqs):
        c0, c1 = layout.seq_chunks[s], layout.seq_chunks[s + 1]
        run = -1
        for c in range(c0, c1):
            if c - c0 < clean_per_video or layout.q_offsets[c + 1] == layout.q_offsets[c]:
                prompt_of_chunk.append(None)
                continue
            r = (c - c0 - clean_per_video) // chunks_per_prompt
            if r != run:
                run = r
                n_prompts += 1
            prompt_of_chunk.append(n_prompts - 1)
    rng = np.random.default_rng(seed)
    lengths = rng.integers(lo, hi + 1, n_prompts)
    return chunk_prompts(prompt_of_chunk, [int(x) for x in lengths])


def tokens_per_chunk(height: int, width: int, frames: int = 24, patch: int = 2) -> int:
    lat_frames = frames // 4
    return lat_frames * (height // 8 // patch) * (width // 8 // patch)


@dataclasses.dataclass(frozen=True)
class Config:
    name: str
    layout: Layout
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    dtype: str            # "bf16" or "fp32"
    gain_kind: str        # "ones" or "uniform" (U(0.5, 1.5))
    seed: int
    eps: float = 1e-6

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.head_dim)


def _configs() -> List[Config]:
    tiny = Config("tiny", layout_from_chunks([[64, 64, 64]]), 2, 1, 64, "fp32", "ones", 1)
    c256 = tokens_per_chunk(256, 256)                       # 1536
    v256 = Config("video256x2", layout_from_chunks([[c256] * 4, [c256] * 4]), 24, 8, 128, "bf16", "uniform", 2)
    stream = Config("streaming", streaming_layout(16, 4, c256), 24, 8, 128, "bf16", "ones", 3)
    c480 = tokens_per_chunk(480, 832)                       # 9360
    v480 = Config("video480x832", layout_from_chunks([[c480] * 16]), 48, 8, 128, "bf16", "ones", 4)
    packed = Config("packed8", layout_from_chunks(packed_chunk_draw(8)), 32, 8, 128, "bf16", "ones", 5)
    return [tiny, v256, stream, v480, packed]


CONFIGS = _configs()


def text_layout(cfg: Config) -> TextLayout:
    """The cross-attention text of a workload (seed = the workload's + 100):
      tiny          chunk 0 clean, chunks 1 and 2 with their own prompts of
                    9..40 tokens (ragged against 32-key tiles);
      video256x2    per video: chunk 0 clean, one prompt per 2 chunks;
      streaming     cached chunks without text, the 4 active chunks one
                    prompt per 2 chunks;
      video480x832  chunks 0, 1 clean, one prompt per 4 chunks;
      packed8       per video: chunk 0 clean (one-chunk videos have no text),
                    one prompt for the rest of the video.
    Prompt lengths are uniform on [64, 512] tokens (tiny: [9, 40])."""
    seed = cfg.seed + 100
    if cfg.name == "tiny":
        return prompt_draw(cfg.layout, 1, 1, seed, 9, 40)
    if cfg.name == "video256x2":
        return prompt_draw(cfg.layout, 1, 2, seed)
    if cfg.name == "streaming":
        return prompt_draw(cfg.layout, 0, 2, seed)
    if cfg.name == "video480x832":
        return prompt_draw(cfg.layout, 2, 4, seed)
    if cfg.name == "packed8":
        return prompt_draw(cfg.layout, 1, 1 << 30, seed)
    raise KeyError(cfg.name)


def get_config(name_or_index) -> Config:
    if isinstance(name_or_index, int):
        return CONFIGS[name_or_index]
    for c in CONFIGS:
        if c.name == name_or_index:
            return c
    raise KeyError(name_or_index)
