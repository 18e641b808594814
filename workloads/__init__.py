"""Seeded synthetic workloads for block-causal attention.

This package holds the chunk layouts of the five benchmark shapes and the seeded
generators of Q, K, V and the QK-norm gains. It holds none of the attention's
arithmetic (no normalisation, no mask, no softmax): both the CPU oracle tests
and the HIP path take their inputs from here, and nothing else is shared.
"""
from .configs import CONFIGS, Layout, get_config, layout_from_chunks, streaming_layout
from .gen import make_inputs

__all__ = ["CONFIGS", "Layout", "get_config", "layout_from_chunks", "streaming_layout", "make_inputs"]
