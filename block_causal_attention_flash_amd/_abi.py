"""ctypes declarations of the C ABI in include/magi_attn.h.

The library is loaded after torch on purpose: libmagi_attn.so needs
libamdhip64.so.7, and the copy torch has already loaded satisfies that
dependency, so torch's streams and device pointers are valid inside it (one
HIP runtime per process).
"""
import ctypes
import os

LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libmagi_attn.so")

MAGI_OK = 0
MAGI_ERR_INVALID_ARG = 1
MAGI_ERR_UNSUPPORTED = 2
MAGI_ERR_NO_MEMORY = 3
MAGI_ERR_HIP = 4

MAGI_DTYPE_BF16 = 0
MAGI_DTYPE_FP32 = 1

MAGI_ATTN_NOALLOC_SCRATCH_BYTES = 256 << 20    # include/magi_attn.h

_i32p = ctypes.POINTER(ctypes.c_int32)


class Layout(ctypes.Structure):
    _fields_ = [
        ("n_seqs", ctypes.c_int32),
        ("seq_chunks", _i32p),
        ("n_chunks", ctypes.c_int32),
        ("q_offsets", _i32p),
        ("kv_offsets", _i32p),
        ("n_q_heads", ctypes.c_int32),
        ("n_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("dtype", ctypes.c_int32),
        ("kv_range", ctypes.c_int32),
        ("last_global", ctypes.c_int32),
    ]


class Text(ctypes.Structure):
    _fields_ = [
        ("t_text", ctypes.c_int32),
        ("text_begin", _i32p),
        ("text_end", _i32p),
    ]


class ParallelIO(ctypes.Structure):
    _fields_ = [
        ("q", ctypes.c_void_p),
        ("k", ctypes.c_void_p),
        ("v", ctypes.c_void_p),
        ("q_gain", ctypes.c_void_p),
        ("k_gain", ctypes.c_void_p),
        ("scale", ctypes.c_float),
        ("out", ctypes.c_void_p),
        ("lse", ctypes.c_void_p),
        ("q_x", ctypes.c_void_p),
        ("k_x", ctypes.c_void_p),
        ("v_x", ctypes.c_void_p),
        ("q_gain_x", ctypes.c_void_p),
        ("k_gain_x", ctypes.c_void_p),
        ("scale_x", ctypes.c_float),
        ("out_x", ctypes.c_void_p),
        ("lse_x", ctypes.c_void_p),
    ]


class BwdIO(ctypes.Structure):
    _fields_ = [(n, ctypes.c_void_p) for n in ("q", "k", "v", "q_gain", "k_gain", "out", "lse", "dout", "dq", "dk",
                                               "dv", "dq_gain", "dk_gain")]


class Stats(ctypes.Structure):
    _fields_ = [
        ("unmasked_pairs", ctypes.c_int64),
        ("full_pairs", ctypes.c_int64),
        ("boundary_pairs", ctypes.c_int64),
        ("empty_pairs", ctypes.c_int64),
        ("executed_pairs", ctypes.c_int64),
        ("tile_q", ctypes.c_int32),
        ("tile_kv", ctypes.c_int32),
        ("heads_per_item", ctypes.c_int32),
        ("n_items", ctypes.c_int32),
    ]


# name -> (restype, argtypes)
SIGNATURES = {
    "magi_attn_plan_create": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(ctypes.c_void_p)]),
    "magi_attn_train_plan_create": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(ctypes.c_void_p)]),
    "magi_attn_cross_train_plan_create": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(Text),
                                                         ctypes.POINTER(ctypes.c_void_p)]),
    "magi_attn_bwd_workspace_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
    "magi_attn_bwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(BwdIO), ctypes.c_float, ctypes.c_float,
                                     ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "magi_attn_cross_plan_create": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(Text),
                                                   ctypes.POINTER(ctypes.c_void_p)]),
    "magi_attn_parallel_plan_create": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(Text),
                                                      ctypes.POINTER(ctypes.c_void_p)]),
    "magi_attn_plan_destroy": (ctypes.c_int, [ctypes.c_void_p]),
    "magi_attn_workspace_size": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ctypes.c_size_t)]),
    "magi_attn_fwd": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                                     ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_size_t,
                                     ctypes.c_void_p]),
    "magi_attn_fwd_noalloc": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_float, ctypes.c_float,
                                             ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p]),
    "magi_attn_fwd_parallel": (ctypes.c_int, [ctypes.c_void_p, ctypes.POINTER(ParallelIO), ctypes.c_float,
                                              ctypes.c_void_p, ctypes.c_size_t, ctypes.c_void_p]),
    "magi_attn_fwd_simple": (ctypes.c_int, [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_void_p, _i32p, ctypes.c_int32, ctypes.c_int32, ctypes.c_int32,
                                            ctypes.c_int32, ctypes.c_int32, ctypes.c_void_p, ctypes.c_void_p,
                                            ctypes.c_float, ctypes.c_float, ctypes.c_void_p]),
    "magi_attn_classify_host": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.c_int32, ctypes.c_int32,
                                               ctypes.POINTER(ctypes.c_int8)]),
    "magi_attn_plan_stats": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(Stats)]),
    "magi_attn_key_classify_host": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.c_int32, ctypes.c_int32,
                                                   ctypes.POINTER(ctypes.c_int8)]),
    "magi_attn_cross_classify_host": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(Text), ctypes.c_int32,
                                                     ctypes.c_int32, ctypes.POINTER(ctypes.c_int8)]),
    "magi_attn_cross_plan_stats": (ctypes.c_int, [ctypes.POINTER(Layout), ctypes.POINTER(Text), ctypes.c_int32,
                                                  ctypes.POINTER(Stats)]),
    "magi_attn_status_str": (ctypes.c_char_p, [ctypes.c_int]),
    "magi_attn_last_error": (ctypes.c_char_p, []),
    "magi_attn_abi_version": (ctypes.c_int, []),
}

_lib = None


def load():
    """Loads the in-tree library (after torch); raises if it was not built."""
    global _lib
    if _lib is not None:
        return _lib
    import torch  # noqa: F401  -- binds libamdhip64.so.7 to torch's copy first
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is missing: build it with `python -c 'import __graft_entry__ as g; g.build()'`"
                           " (or python block_causal_attention_flash_amd/build.py)")
    lib = ctypes.CDLL(LIB_PATH)
    for name, (res, args) in SIGNATURES.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args
    _lib = lib
    return lib
