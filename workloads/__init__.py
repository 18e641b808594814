"""Seeded synthetic workloads for block-causal attention.

This package holds the chunk layouts of the five benchmark shapes, the
chunk-wise prompt layouts of their text streams, and the seeded generators of
Q, K, V, the text K/V and the QK-norm gains. It holds none of the attention's
arithmetic (no normalisation, no mask, no softmax): both the CPU oracle tests
and the HIP path take their inputs from here, and nothing else is shared.
"""
from .configs import (CONFIGS, Layout, TextLayout, chunk_prompts, get_config, layout_from_chunks, prompt_draw,
                      streaming_layout, text_layout)
from .gen import make_inputs, make_text_inputs

__all__ = ["CONFIGS", "Layout", "TextLayout", "chunk_prompts", "get_config", "layout_from_chunks", "prompt_draw",
           "streaming_layout", "text_layout", "make_inputs", "make_text_inputs"]
