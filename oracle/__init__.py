"""CPU oracle (fp64) of block-causal QK-norm GQA attention, its backward, and
the text cross-attention that runs beside it.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
CPU-baseline leg of bench.py, never by the product library or its binding.
"""
from .backward import attention_backward, cross_attention_backward, cross_dkv_keys, cross_dq_rows, dkv_keys, dq_rows
from .cross import cross_attention, cross_attention_loops, text_mask, text_pairs
from .dense import (attention, attention_loops, attention_probs, block_causal_mask,
                    chunk_video_ids, rms_norm, token_chunk_ids, unmasked_pairs)

__all__ = ["attention", "attention_backward", "attention_loops", "cross_attention_backward", "cross_dkv_keys",
           "cross_dq_rows", "dkv_keys", "dq_rows", "attention_probs", "block_causal_mask",
           "chunk_video_ids", "cross_attention", "cross_attention_loops", "rms_norm", "text_mask",
           "text_pairs", "token_chunk_ids", "unmasked_pairs"]
