"""CPU oracle (fp64) of block-causal QK-norm GQA attention.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the product library or its binding.
"""
from .dense import (attention, attention_loops, attention_probs, block_causal_mask,
                    chunk_video_ids, rms_norm, token_chunk_ids, unmasked_pairs)

__all__ = ["attention", "attention_loops", "attention_probs", "block_causal_mask",
           "chunk_video_ids", "rms_norm", "token_chunk_ids", "unmasked_pairs"]
