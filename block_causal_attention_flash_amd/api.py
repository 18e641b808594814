"""Argument marshalling for the C ABI (include/magi_attn.h); no computation here."""
from __future__ import annotations

import ctypes
from typing import Optional, Sequence, Tuple

import numpy as np

from . import _abi

_DTYPES = {"bf16": _abi.MAGI_DTYPE_BF16, "fp32": _abi.MAGI_DTYPE_FP32}


class MagiAttnError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status
        self.message = message


def _check(lib, status: int):
    if status != _abi.MAGI_OK:
        msg = lib.magi_attn_last_error().decode(errors="replace")
        raise MagiAttnError(status, msg or lib.magi_attn_status_str(status).decode())


def _arr(x) -> np.ndarray:
    return np.ascontiguousarray(np.asarray(x, dtype=np.int32))


class _LayoutArgs:
    """Keeps the host offset arrays alive for the duration of a call."""

    def __init__(self, q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range=0, last_global=0):
        self.q = _arr(q_offsets)
        self.kv = None if kv_offsets is None else _arr(kv_offsets)
        n_chunks = len(self.q) - 1
        self.seq = _arr([0, n_chunks] if seq_chunks is None else seq_chunks)
        p = lambda a: None if a is None else a.ctypes.data_as(_abi._i32p)  # noqa: E731
        dt = _DTYPES[dtype] if isinstance(dtype, str) else int(dtype)
        self.struct = _abi.Layout(len(self.seq) - 1, p(self.seq), n_chunks, p(self.q), p(self.kv),
                                  int(n_q_heads), int(n_kv_heads), int(head_dim), dt, int(kv_range),
                                  int(last_global))

    def ptr(self):
        return ctypes.byref(self.struct)


class _TextArgs:
    """Keeps the host text-range arrays alive for the duration of a call."""

    def __init__(self, text_begin, text_end, t_text):
        self.b = _arr(text_begin)
        self.e = _arr(text_end)
        self.struct = _abi.Text(int(t_text), self.b.ctypes.data_as(_abi._i32p), self.e.ctypes.data_as(_abi._i32p))

    def ptr(self):
        return ctypes.byref(self.struct)


def magi_attn_abi_version() -> int:
    return _abi.load().magi_attn_abi_version()


def magi_attn_plan_stats(q_offsets, kv_offsets=None, seq_chunks=None, n_q_heads=1, n_kv_heads=1, head_dim=128,
                         dtype="bf16", kv_range=0, last_global=0) -> dict:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    st = _abi.Stats()
    _check(lib, lib.magi_attn_plan_stats(la.ptr(), ctypes.byref(st)))
    return {name: getattr(st, name) for name, _ in _abi.Stats._fields_}


def magi_attn_classify_host(q_offsets, kv_offsets=None, seq_chunks=None, bm=128, bn=64, n_q_heads=1, n_kv_heads=1,
                            head_dim=128, dtype="bf16", kv_range=0, last_global=0) -> np.ndarray:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    tq = int(la.q[-1])
    tk = int((la.kv if la.kv is not None else la.q)[-1])
    n_qt, n_kt = -(-tq // bm), -(-tk // bn)
    cls = np.zeros((max(n_qt, 0), max(n_kt, 0)), dtype=np.int8)
    _check(lib, lib.magi_attn_classify_host(la.ptr(), bm, bn, cls.ctypes.data_as(ctypes.POINTER(ctypes.c_int8))))
    return cls


def magi_attn_key_classify_host(q_offsets, kv_offsets=None, seq_chunks=None, bk=128, bt=32, n_q_heads=1, n_kv_heads=1,
                                head_dim=128, dtype="bf16", kv_range=0, last_global=0) -> np.ndarray:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    tq = int(la.q[-1])
    tk = int((la.kv if la.kv is not None else la.q)[-1])
    cls = np.zeros((max(-(-tk // bk), 0), max(-(-tq // bt), 0)), dtype=np.int8)
    _check(lib, lib.magi_attn_key_classify_host(la.ptr(), bk, bt, cls.ctypes.data_as(ctypes.POINTER(ctypes.c_int8))))
    return cls


def magi_attn_cross_classify_host(q_offsets, text_begin, text_end, t_text, bm=128, bn=64, kv_offsets=None,
                                  seq_chunks=None, n_q_heads=1, n_kv_heads=1, head_dim=128, dtype="bf16",
                                  kv_range=0, last_global=0) -> np.ndarray:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    ta = _TextArgs(text_begin, text_end, t_text)
    n_qt, n_kt = -(-int(la.q[-1]) // bm), -(-int(t_text) // bn)
    cls = np.zeros((max(n_qt, 0), max(n_kt, 0)), dtype=np.int8)
    _check(lib, lib.magi_attn_cross_classify_host(la.ptr(), ta.ptr(), bm, bn,
                                                  cls.ctypes.data_as(ctypes.POINTER(ctypes.c_int8))))
    return cls


def magi_attn_cross_plan_stats(q_offsets, text_begin, text_end, t_text, kv_offsets=None, seq_chunks=None,
                               n_q_heads=1, n_kv_heads=1, head_dim=128, dtype="bf16", kv_range=0, last_global=0,
                               with_self=False) -> dict:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    ta = _TextArgs(text_begin, text_end, t_text)
    st = _abi.Stats()
    _check(lib, lib.magi_attn_cross_plan_stats(la.ptr(), ta.ptr(), int(bool(with_self)), ctypes.byref(st)))
    return {name: getattr(st, name) for name, _ in _abi.Stats._fields_}


def magi_attn_plan_create(q_offsets, kv_offsets=None, seq_chunks=None, n_q_heads=1, n_kv_heads=1, head_dim=128,
                          dtype="bf16", kv_range=0, last_global=0) -> int:
    """Returns the opaque plan handle (an integer address)."""
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    h = ctypes.c_void_p()
    _check(lib, lib.magi_attn_plan_create(la.ptr(), ctypes.byref(h)))
    return h.value


def magi_attn_train_plan_create(q_offsets, kv_offsets=None, seq_chunks=None, n_q_heads=1, n_kv_heads=1, head_dim=128,
                                dtype="bf16", kv_range=0, last_global=0) -> int:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    h = ctypes.c_void_p()
    _check(lib, lib.magi_attn_train_plan_create(la.ptr(), ctypes.byref(h)))
    return h.value


def magi_attn_cross_train_plan_create(q_offsets, text_begin, text_end, t_text, kv_offsets=None, seq_chunks=None,
                                      n_q_heads=1, n_kv_heads=1, head_dim=128, dtype="bf16", kv_range=0,
                                      last_global=0) -> int:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    ta = _TextArgs(text_begin, text_end, t_text)
    h = ctypes.c_void_p()
    _check(lib, lib.magi_attn_cross_train_plan_create(la.ptr(), ta.ptr(), ctypes.byref(h)))
    return h.value


def magi_attn_bwd_workspace_size(handle: int) -> int:
    lib = _abi.load()
    n = ctypes.c_size_t()
    _check(lib, lib.magi_attn_bwd_workspace_size(handle, ctypes.byref(n)))
    return n.value


def magi_attn_bwd(handle: int, q, k, v, out, lse, dout, q_gain=None, k_gain=None, rms_eps: float = 1e-6,
                  scale: Optional[float] = None, dq=None, dk=None, dv=None, dq_gain=None, dk_gain=None,
                  workspace=None, stream=None):
    """Enqueues the backward on `stream`: the gradients with respect to q, k,
    v and both gains for the upstream gradient dout of out. Returns
    (dq, dk, dv, dq_gain, dk_gain)."""
    import torch
    lib = _abi.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse), ("dout", dout)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    d = q.shape[-1]
    dev = q.device
    sc = (1.0 / d ** 0.5) if scale is None else float(scale)
    with _alloc_on(stream):
        dq = torch.empty_like(q) if dq is None else dq
        dk = torch.empty_like(k) if dk is None else dk
        dv = torch.empty_like(v) if dv is None else dv
        dq_gain = torch.empty(d, dtype=torch.float32, device=dev) if dq_gain is None else dq_gain
        dk_gain = torch.empty(d, dtype=torch.float32, device=dev) if dk_gain is None else dk_gain
        qg = _gain(q_gain, d, dev)
        kg = _gain(k_gain, d, dev)
        if workspace is None:                          # (the library checks a given workspace's size)
            workspace = torch.empty(max(magi_attn_bwd_workspace_size(handle), 16), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
        io = _abi.BwdIO(*(t.data_ptr() for t in (q, k, v, qg, kg, out, lse, dout, dq, dk, dv, dq_gain, dk_gain)))
        _check(lib, lib.magi_attn_bwd(handle, ctypes.byref(io), float(rms_eps), sc, workspace.data_ptr(), ws_bytes,
                                      _stream_ptr(stream, dev)))
    return dq, dk, dv, dq_gain, dk_gain


def magi_attn_cross_plan_create(q_offsets, text_begin, text_end, t_text, kv_offsets=None, seq_chunks=None,
                                n_q_heads=1, n_kv_heads=1, head_dim=128, dtype="bf16", kv_range=0, last_global=0) -> int:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    ta = _TextArgs(text_begin, text_end, t_text)
    h = ctypes.c_void_p()
    _check(lib, lib.magi_attn_cross_plan_create(la.ptr(), ta.ptr(), ctypes.byref(h)))
    return h.value


def magi_attn_parallel_plan_create(q_offsets, text_begin, text_end, t_text, kv_offsets=None, seq_chunks=None,
                                   n_q_heads=1, n_kv_heads=1, head_dim=128, dtype="bf16", kv_range=0, last_global=0) -> int:
    lib = _abi.load()
    la = _LayoutArgs(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
    ta = _TextArgs(text_begin, text_end, t_text)
    h = ctypes.c_void_p()
    _check(lib, lib.magi_attn_parallel_plan_create(la.ptr(), ta.ptr(), ctypes.byref(h)))
    return h.value


def magi_attn_plan_destroy(handle: int) -> None:
    lib = _abi.load()
    _check(lib, lib.magi_attn_plan_destroy(handle))


def magi_attn_workspace_size(handle: int) -> int:
    lib = _abi.load()
    n = ctypes.c_size_t()
    _check(lib, lib.magi_attn_workspace_size(handle, ctypes.byref(n)))
    return n.value


def _alloc_on(stream):
    """Context in which the wrappers allocate their temporaries and default
    outputs: the caller's `stream`, so that torch's caching allocator ties
    that memory to the stream the kernels read and write it on (it is reused
    only after the stream's work, never under it). None: the current stream."""
    import contextlib
    import torch
    return contextlib.nullcontext() if stream is None else torch.cuda.stream(stream)


def _stream_ptr(stream, device):
    import torch
    s = torch.cuda.current_stream(device) if stream is None else stream
    return ctypes.c_void_p(s.cuda_stream)


def _gain(g, d, device):
    import torch
    if g is None:
        return torch.ones(d, dtype=torch.float32, device=device)
    g = g.to(device=device, dtype=torch.float32).contiguous()
    if g.shape != (d,):
        raise ValueError(f"gain must have shape ({d},)")
    return g


def magi_attn_fwd(handle: int, q, k, v, q_gain=None, k_gain=None, rms_eps: float = 1e-6,
                  scale: Optional[float] = None, out=None, lse=None, workspace=None, stream=None):
    """Enqueues the forward on `stream` (default: torch's current stream).
    q [T_q,H_q,d], k/v [T_k,H_kv,d] on the GPU; `workspace` is a device
    tensor of at least magi_attn_workspace_size(handle) bytes (allocated here
    when None). Returns (out, lse)."""
    import torch
    lib = _abi.load()
    for name, t in (("q", q), ("k", k), ("v", v)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    d = q.shape[-1]
    sc = (1.0 / d ** 0.5) if scale is None else float(scale)
    with _alloc_on(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
        qg = _gain(q_gain, d, q.device)
        kg = _gain(k_gain, d, q.device)
        if workspace is None:                          # (the library checks a given workspace's size)
            workspace = torch.empty(max(magi_attn_workspace_size(handle), 16), dtype=torch.uint8, device=q.device)
        ws_bytes = workspace.numel() * workspace.element_size()
        _check(lib, lib.magi_attn_fwd(handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), qg.data_ptr(), kg.data_ptr(),
                                      float(rms_eps), sc, out.data_ptr(), lse.data_ptr(), workspace.data_ptr(),
                                      ws_bytes, _stream_ptr(stream, q.device)))
    return out, lse


def magi_attn_fwd_noalloc(handle: int, q, k, v, q_gain, k_gain, rms_eps: float, scale: float, out, lse,
                          stream=None):
    """magi_attn_fwd with the library's static device scratch as the
    workspace: nothing is allocated here or in the library, so every tensor,
    the gains included (fp32, on the device), must be given. Plans whose
    workspace exceeds MAGI_ATTN_NOALLOC_SCRATCH_BYTES are refused. Calls that
    overlap on one GPU share the scratch and must not run concurrently."""
    lib = _abi.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("lse", lse)):
        if t is None or not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    for name, g in (("q_gain", q_gain), ("k_gain", k_gain)):
        if g is None or not g.is_cuda or not g.is_contiguous() or str(g.dtype) != "torch.float32":
            raise ValueError(f"{name} must be a contiguous fp32 GPU tensor")
    _check(lib, lib.magi_attn_fwd_noalloc(handle, q.data_ptr(), k.data_ptr(), v.data_ptr(), q_gain.data_ptr(),
                                          k_gain.data_ptr(), float(rms_eps), float(scale), out.data_ptr(),
                                          lse.data_ptr(), _stream_ptr(stream, q.device)))
    return out, lse


def magi_attn_fwd_parallel(handle: int, q, k, v, q_x, k_x, v_x, q_gain=None, k_gain=None, q_gain_x=None,
                           k_gain_x=None, rms_eps: float = 1e-6, scale: Optional[float] = None,
                           scale_x: Optional[float] = None, out=None, lse=None, out_x=None, lse_x=None,
                           workspace=None, stream=None):
    """Enqueues both attentions of a parallel plan on `stream`: the
    self-attention of q over k/v and the cross-attention of q_x over the text
    k_x/v_x. Returns (out, lse, out_x, lse_x)."""
    import torch
    lib = _abi.load()
    for name, t in (("q", q), ("k", k), ("v", v), ("q_x", q_x), ("k_x", k_x), ("v_x", v_x)):
        if not t.is_cuda or not t.is_contiguous():
            raise ValueError(f"{name} must be a contiguous GPU tensor")
    d = q.shape[-1]
    dev = q.device
    lse_shape = (q.shape[1], q.shape[0])
    sc = (1.0 / d ** 0.5) if scale is None else float(scale)
    scx = (1.0 / d ** 0.5) if scale_x is None else float(scale_x)
    with _alloc_on(stream):
        out = torch.empty_like(q) if out is None else out
        lse = torch.empty(lse_shape, dtype=torch.float32, device=dev) if lse is None else lse
        out_x = torch.empty_like(q_x) if out_x is None else out_x
        lse_x = torch.empty(lse_shape, dtype=torch.float32, device=dev) if lse_x is None else lse_x
        gains = [_gain(g, d, dev) for g in (q_gain, k_gain, q_gain_x, k_gain_x)]
        if workspace is None:                          # (the library checks a given workspace's size)
            workspace = torch.empty(max(magi_attn_workspace_size(handle), 16), dtype=torch.uint8, device=dev)
        ws_bytes = workspace.numel() * workspace.element_size()
        io = _abi.ParallelIO(q.data_ptr(), k.data_ptr(), v.data_ptr(), gains[0].data_ptr(), gains[1].data_ptr(), sc,
                             out.data_ptr(), lse.data_ptr(), q_x.data_ptr(), k_x.data_ptr(), v_x.data_ptr(),
                             gains[2].data_ptr(), gains[3].data_ptr(), scx, out_x.data_ptr(), lse_x.data_ptr())
        _check(lib, lib.magi_attn_fwd_parallel(handle, ctypes.byref(io), float(rms_eps), workspace.data_ptr(),
                                               ws_bytes, _stream_ptr(stream, dev)))
    return out, lse, out_x, lse_x


def magi_attn_fwd_simple(q, k, v, chunk_offsets: Sequence[int], q_gain=None, k_gain=None, rms_eps: float = 1e-6,
                         scale: Optional[float] = None, out=None, lse=None, stream=None):
    """One video of self-attention with q/kv offsets = chunk_offsets."""
    import torch
    lib = _abi.load()
    offs = _arr(chunk_offsets)
    d = q.shape[-1]
    dt = {torch.bfloat16: _abi.MAGI_DTYPE_BF16, torch.float32: _abi.MAGI_DTYPE_FP32}[q.dtype]
    sc = (1.0 / d ** 0.5) if scale is None else float(scale)
    with _alloc_on(stream):
        if out is None:
            out = torch.empty_like(q)
        if lse is None:
            lse = torch.empty((q.shape[1], q.shape[0]), dtype=torch.float32, device=q.device)
        qg = _gain(q_gain, d, q.device)
        kg = _gain(k_gain, d, q.device)
        _check(lib, lib.magi_attn_fwd_simple(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(),
                                             lse.data_ptr(), offs.ctypes.data_as(_abi._i32p), len(offs) - 1,
                                             q.shape[1], k.shape[1], d, dt, qg.data_ptr(), kg.data_ptr(),
                                             float(rms_eps), sc, _stream_ptr(stream, q.device)))
    return out, lse


class Plan:
    """Owns a plan handle for one layout; call() runs the forward."""

    def __init__(self, q_offsets, kv_offsets=None, seq_chunks=None, n_q_heads=1, n_kv_heads=1, head_dim=128,
                 dtype="bf16", kv_range=0, last_global=0):
        self.layout = dict(q_offsets=list(map(int, q_offsets)),
                           kv_offsets=None if kv_offsets is None else list(map(int, kv_offsets)),
                           seq_chunks=None if seq_chunks is None else list(map(int, seq_chunks)),
                           n_q_heads=n_q_heads, n_kv_heads=n_kv_heads, head_dim=head_dim, dtype=dtype,
                           kv_range=int(kv_range), last_global=int(last_global))
        self.n_q_heads, self.n_kv_heads, self.head_dim, self.dtype = n_q_heads, n_kv_heads, head_dim, dtype
        self.t_q = int(self.layout["q_offsets"][-1])
        kv = self.layout["kv_offsets"] or self.layout["q_offsets"]
        self.t_k = int(kv[-1])
        self.handle = None
        self.handle = self._create()

    def _create(self) -> int:
        return magi_attn_plan_create(**self.layout)

    @classmethod
    def from_layout(cls, layout, n_q_heads, n_kv_heads, head_dim, dtype="bf16"):
        return cls(layout.q_offsets, layout.kv_offsets, layout.seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype,
                   getattr(layout, "kv_range", 0), getattr(layout, "last_global", 0))

    def stats(self) -> dict:
        return magi_attn_plan_stats(**self.layout)

    def workspace_size(self) -> int:
        return magi_attn_workspace_size(self.handle)

    def _check(self, q, k, v, t_k, out, lse):
        import torch
        want = torch.bfloat16 if self.dtype == "bf16" else torch.float32
        if q.dtype != want or k.dtype != want or v.dtype != want:
            raise ValueError(f"q, k, v must be {want}")
        if tuple(q.shape) != (self.t_q, self.n_q_heads, self.head_dim):
            raise ValueError(f"q must have shape {(self.t_q, self.n_q_heads, self.head_dim)}")
        if tuple(k.shape) != (t_k, self.n_kv_heads, self.head_dim) or k.shape != v.shape:
            raise ValueError(f"k and v must have shape {(t_k, self.n_kv_heads, self.head_dim)}")
        if out is not None and (out.shape != q.shape or out.dtype != want or not out.is_contiguous()):
            raise ValueError("out must match q")
        if lse is not None and (tuple(lse.shape) != (self.n_q_heads, self.t_q) or lse.dtype != torch.float32):
            raise ValueError("lse must be float32 [H_q, T_q]")

    def __call__(self, q, k, v, q_gain=None, k_gain=None, rms_eps=1e-6, scale=None, out=None, lse=None,
                 workspace=None, stream=None):
        self._check(q, k, v, self.t_k, out, lse)
        return magi_attn_fwd(self.handle, q, k, v, q_gain, k_gain, rms_eps, scale, out, lse, workspace, stream)

    def close(self):
        if self.handle:
            magi_attn_plan_destroy(self.handle)
            self.handle = None

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


class CrossPlan(Plan):
    """Plan of the text cross-attention alone: call(q, k_text, v_text, ...)
    with the cross-attention's gains and temperature."""

    def __init__(self, q_offsets, text_begin, text_end, t_text, kv_offsets=None, seq_chunks=None, n_q_heads=1,
                 n_kv_heads=1, head_dim=128, dtype="bf16", kv_range=0, last_global=0):
        self.text = dict(text_begin=list(map(int, text_begin)), text_end=list(map(int, text_end)),
                         t_text=int(t_text))
        super().__init__(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)
        self.t_k = self.text["t_text"]

    def _create(self) -> int:
        return magi_attn_cross_plan_create(**self.layout, **self.text)

    @classmethod
    def from_layout(cls, layout, text, n_q_heads, n_kv_heads, head_dim, dtype="bf16"):
        return cls(layout.q_offsets, text.begin, text.end, text.t_text, layout.kv_offsets, layout.seq_chunks,
                   n_q_heads, n_kv_heads, head_dim, dtype, getattr(layout, "kv_range", 0),
                   getattr(layout, "last_global", 0))

    def stats(self) -> dict:
        return magi_attn_cross_plan_stats(**self.layout, **self.text)


class ParallelPlan(Plan):
    """Plan of the parallel attention block: the self-attention of a layout
    and the cross-attention of a text, run as one pass by call()."""

    def __init__(self, q_offsets, text_begin, text_end, t_text, kv_offsets=None, seq_chunks=None, n_q_heads=1,
                 n_kv_heads=1, head_dim=128, dtype="bf16", kv_range=0, last_global=0):
        self.text = dict(text_begin=list(map(int, text_begin)), text_end=list(map(int, text_end)),
                         t_text=int(t_text))
        super().__init__(q_offsets, kv_offsets, seq_chunks, n_q_heads, n_kv_heads, head_dim, dtype, kv_range, last_global)

    def _create(self) -> int:
        return magi_attn_parallel_plan_create(**self.layout, **self.text)

    @classmethod
    def from_layout(cls, layout, text, n_q_heads, n_kv_heads, head_dim, dtype="bf16"):
        return cls(layout.q_offsets, text.begin, text.end, text.t_text, layout.kv_offsets, layout.seq_chunks,
                   n_q_heads, n_kv_heads, head_dim, dtype, getattr(layout, "kv_range", 0),
                   getattr(layout, "last_global", 0))

    def stats(self) -> dict:
        return magi_attn_cross_plan_stats(**self.layout, **self.text, with_self=True)

    def __call__(self, q, k, v, k_x, v_x, q_x=None, q_gain=None, k_gain=None, q_gain_x=None, k_gain_x=None,
                 rms_eps=1e-6, scale=None, scale_x=None, out=None, lse=None, out_x=None, lse_x=None, workspace=None,
                 stream=None):
        q_x = q if q_x is None else q_x
        self._check(q, k, v, self.t_k, out, lse)
        self._check(q_x, k_x, v_x, self.text["t_text"], out_x, lse_x)
        return magi_attn_fwd_parallel(self.handle, q, k, v, q_x, k_x, v_x, q_gain, k_gain, q_gain_x, k_gain_x,
                                      rms_eps, scale, scale_x, out, lse, out_x, lse_x, workspace, stream)


class _Backward:
    """backward() of a training plan: the gradients from the forward's out
    and lse (keys of the plan's key stream: the video's, or the text's)."""

    def bwd_workspace_size(self) -> int:
        return magi_attn_bwd_workspace_size(self.handle)

    def backward(self, q, k, v, out, lse, dout, q_gain=None, k_gain=None, rms_eps=1e-6, scale=None, dq=None, dk=None,
                 dv=None, dq_gain=None, dk_gain=None, workspace=None, stream=None):
        self._check(q, k, v, self.t_k, out, lse)
        if dout.shape != q.shape or dout.dtype != q.dtype:
            raise ValueError("dout must match q")
        return magi_attn_bwd(self.handle, q, k, v, out, lse, dout, q_gain, k_gain, rms_eps, scale, dq, dk, dv, dq_gain,
                             dk_gain, workspace, stream)


class TrainPlan(_Backward, Plan):
    """A self-attention plan that also runs the backward: call() is the
    forward, backward() the gradients from the forward's out and lse."""

    def _create(self) -> int:
        return magi_attn_train_plan_create(**self.layout)


class CrossTrainPlan(_Backward, CrossPlan):
    """A cross-attention plan that also runs the backward: call(q, k_text,
    v_text, ...) is the forward, backward(q, k_text, v_text, out, lse, dout,
    ...) the gradients, dk and dv over the text tokens."""

    def _create(self) -> int:
        return magi_attn_cross_train_plan_create(**self.layout, **self.text)
