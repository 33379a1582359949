"""ctypes binding of libinfllm2.so (C ABI declared in include/infllm2.h).

Argument marshalling only: tensors are checked for device, dtype, shape and contiguity, then
their device pointers and the current HIP stream are handed to the library.
"""
from __future__ import annotations

import ctypes
import math
import os
import re
from dataclasses import dataclass
from typing import Optional, Sequence

import numpy as np

F32 = 0
BF16 = 1

_PKG = os.path.dirname(os.path.abspath(__file__))
_ROOT = os.path.dirname(_PKG)
_HEADER = os.path.join(_ROOT, "include", "infllm2.h")


def library_path() -> str:
    return os.environ.get("INFLLM2_LIB", os.path.join(_PKG, "libinfllm2.so"))


class InfLLM2Error(RuntimeError):
    def __init__(self, status: int, func: str, detail: str):
        super().__init__(f"{func} failed with status {status}: {detail}")
        self.status = status


class _CParams(ctypes.Structure):
    _fields_ = [("num_q_heads", ctypes.c_int32), ("num_kv_heads", ctypes.c_int32),
                ("head_dim", ctypes.c_int32), ("block_size", ctypes.c_int32),
                ("kernel_size", ctypes.c_int32), ("kernel_stride", ctypes.c_int32),
                ("topk", ctypes.c_int32), ("num_init_blocks", ctypes.c_int32),
                ("num_local_blocks", ctypes.c_int32), ("softmax_scale", ctypes.c_float),
                ("dtype", ctypes.c_int32), ("score_mode", ctypes.c_int32)]


_I64P = ctypes.POINTER(ctypes.c_int64)
_I32P = ctypes.POINTER(ctypes.c_int32)


class _CSeqs(ctypes.Structure):
    _fields_ = [("num_seqs", ctypes.c_int32), ("max_q_len", ctypes.c_int32),
                ("max_kv_len", ctypes.c_int32), ("q_rows", ctypes.c_int32),
                ("q_start", ctypes.c_void_p), ("q_len", ctypes.c_void_p),
                ("q_pos0", ctypes.c_void_p), ("kv_start", ctypes.c_void_p),
                ("kv_len", ctypes.c_void_p), ("kc_start", ctypes.c_void_p)]


_lib = None


def _declare(lib):
    P, S = ctypes.POINTER(_CParams), ctypes.POINTER(_CSeqs)
    vp, st = ctypes.c_void_p, ctypes.c_int
    sig = {
        "infllm2_compress_kernels": (st, [P, S, vp, vp, vp, vp]),
        "infllm2_block_scores": (st, [P, S, vp, vp, vp, ctypes.c_int32, vp]),
        "infllm2_topk_select": (st, [P, S, vp, ctypes.c_int32, vp, vp]),
        "infllm2_sparse_attn_prefill": (st, [P, S, vp, vp, vp, vp, vp, vp, vp]),
        "infllm2_decode_workspace_size": (ctypes.c_size_t, [P, ctypes.c_int32, ctypes.c_int32]),
        "infllm2_sparse_attn_decode": (st, [P, S, vp, vp, vp, vp, ctypes.c_int32, vp,
                                            ctypes.c_size_t, vp, vp, vp]),
        "infllm2_decode_step": (st, [P, S, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp,
                                     ctypes.c_int32, vp, ctypes.c_size_t, vp, vp, vp]),
        "infllm2_sliding_window_attn": (st, [P, S, ctypes.c_int32, vp, vp, vp, vp, vp, vp]),
        "infllm2_decode_step_noalloc": (st, [P, S, vp, vp, vp, vp, vp, vp, ctypes.c_int32, vp,
                                             ctypes.c_int32, vp, vp, vp]),
        "infllm2_backward_workspace_size": (ctypes.c_size_t, [P, S]),
        "infllm2_sparse_attn_backward": (st, [P, S, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              ctypes.c_size_t, vp]),
        "infllm2_status_string": (ctypes.c_char_p, [st]),
        "infllm2_last_error": (ctypes.c_char_p, []),
        "infllm2_version": (ctypes.c_int32, []),
    }
    for name, (res, args) in sig.items():
        fn = getattr(lib, name)
        fn.restype = res
        fn.argtypes = args


def load_library():
    """Load (once) and return the ctypes handle.  Raises if the library is missing."""
    global _lib
    if _lib is None:
        path = library_path()
        if not os.path.exists(path):
            raise ImportError(f"libinfllm2 not built: {path} is missing "
                              "(python -m block_sparse_long_semantic_amd.build)")
        lib = ctypes.CDLL(path)
        _declare(lib)
        _lib = lib
    return _lib


def _header_symbols() -> list:
    with open(_HEADER) as f:
        text = f.read()
    return sorted(set(re.findall(r"\b(infllm2_[a-z_]+)\s*\(", text)))


EXPORTED_SYMBOLS = _header_symbols()


def version() -> int:
    return int(load_library().infllm2_version())


# ----------------------------------------------------------------------------- metadata

@dataclass
class Params:
    num_q_heads: int
    num_kv_heads: int
    head_dim: int
    block_size: int = 64
    kernel_size: int = 32
    kernel_stride: int = 16
    topk: int = 96
    num_init_blocks: int = 1
    num_local_blocks: int = 2
    softmax_scale: float = 0.0
    dtype: int = BF16
    score_mode: int = 0

    @staticmethod
    def from_any(p) -> "Params":
        if isinstance(p, Params):
            return p
        dt = getattr(p, "dtype")
        if isinstance(dt, str):
            dt = {"bf16": BF16, "f32": F32}[dt]
        return Params(p.num_q_heads, p.num_kv_heads, p.head_dim, p.block_size, p.kernel_size,
                      p.kernel_stride, p.topk, p.num_init_blocks, p.num_local_blocks,
                      float(getattr(p, "softmax_scale", 0.0)), int(dt),
                      int(getattr(p, "score_mode", 0)))

    @property
    def scale(self) -> float:
        return self.softmax_scale if self.softmax_scale > 0 else 1.0 / math.sqrt(self.head_dim)

    def c(self) -> _CParams:
        return _CParams(self.num_q_heads, self.num_kv_heads, self.head_dim, self.block_size,
                        self.kernel_size, self.kernel_stride, self.topk, self.num_init_blocks,
                        self.num_local_blocks, self.softmax_scale, self.dtype, self.score_mode)


class Seqs:
    """Sequence metadata (the header gives every field's meaning): the per-sequence arrays, kept
    on the host and copied to the device (one packed buffer per device) where the library's
    kernels read them, and the host bounds num_seqs, max_q_len, max_kv_len and q_rows, which
    default to the arrays' own maxima.  Seqs.on_device() wraps arrays that already live on the
    device (no host copy): the caller may rewrite them there between calls, e.g. for the next
    decoding step of a captured graph, within the bounds."""

    def __init__(self, q_start, q_len, q_pos0, kv_start, kv_len, kc_start=None, *,
                 max_q_len: Optional[int] = None, max_kv_len: Optional[int] = None,
                 q_rows: Optional[int] = None):
        self.q_start = np.ascontiguousarray(q_start, dtype=np.int64)
        self.q_len = np.ascontiguousarray(q_len, dtype=np.int32)
        self.q_pos0 = np.ascontiguousarray(q_pos0, dtype=np.int32)
        self.kv_start = np.ascontiguousarray(kv_start, dtype=np.int64)
        self.kv_len = np.ascontiguousarray(kv_len, dtype=np.int32)
        self.kc_start = None if kc_start is None else np.ascontiguousarray(kc_start, dtype=np.int64)
        n = len(self.q_len)
        for a in (self.q_start, self.q_pos0, self.kv_start, self.kv_len):
            if len(a) != n:
                raise ValueError("sequence metadata arrays differ in length")
        if self.kc_start is not None and len(self.kc_start) != n:
            raise ValueError("sequence metadata arrays differ in length")
        self.max_q_len = int(self.q_len.max()) if max_q_len is None and n else int(max_q_len or 0)
        self.max_kv_len = int(self.kv_len.max()) if max_kv_len is None and n else int(max_kv_len or 0)
        self.q_rows = (int((self.q_start + self.q_len).max()) if q_rows is None and n
                       else int(q_rows or 0))
        self._n = n
        self._dev = {}          # device -> (packed buffer, pointers)
        self._device_arrays = None

    @staticmethod
    def on_device(q_start, q_len, q_pos0, kv_start, kv_len, kc_start, *, max_q_len: int,
                  max_kv_len: int, q_rows: int) -> "Seqs":
        """Metadata given as device tensors (int64 starts, int32 lengths and positions; kc_start
        may be None) with explicit host bounds."""
        torch = _torch()
        want = [(q_start, torch.int64), (q_len, torch.int32), (q_pos0, torch.int32),
                (kv_start, torch.int64), (kv_len, torch.int32)]
        if kc_start is not None:
            want.append((kc_start, torch.int64))
        n = int(q_len.numel())
        for t, dt in want:
            if t.device.type != "cuda" or t.dtype != dt or not t.is_contiguous() or t.numel() != n:
                raise ValueError("device metadata must be contiguous device tensors of num_seqs "
                                 "entries (int64 starts, int32 lengths and positions)")
        obj = Seqs.__new__(Seqs)
        obj.q_start = obj.q_len = obj.q_pos0 = obj.kv_start = obj.kv_len = obj.kc_start = None
        obj.max_q_len, obj.max_kv_len, obj.q_rows = int(max_q_len), int(max_kv_len), int(q_rows)
        obj._n = n
        obj._dev = {}
        obj._device_arrays = (q_start, q_len, q_pos0, kv_start, kv_len, kc_start)
        return obj

    @property
    def num_seqs(self) -> int:
        return int(self._n)

    @property
    def total_q_rows(self) -> int:
        return int(self.q_rows)

    @staticmethod
    def packed_prefill(seq_lens: Sequence[int], kc_start: Optional[Sequence[int]] = None,
                       kernel_size: int = 32, kernel_stride: int = 16) -> "Seqs":
        lens = np.asarray(seq_lens, dtype=np.int64)
        starts = np.concatenate([[0], np.cumsum(lens)[:-1]]).astype(np.int64)
        if kc_start is None:
            nk = np.array([0 if L < kernel_size else (L - kernel_size) // kernel_stride + 1
                           for L in lens], dtype=np.int64)
            kc_start = np.concatenate([[0], np.cumsum(nk)[:-1]])
        return Seqs(starts, lens, np.zeros(len(lens)), starts, lens, kc_start)

    @staticmethod
    def decode(kv_len: Sequence[int], max_len: int, max_kernels: int) -> "Seqs":
        kv = np.asarray(kv_len, dtype=np.int64)
        n = len(kv)
        return Seqs(np.arange(n), np.ones(n), kv - 1, np.arange(n) * max_len, kv,
                    np.arange(n) * max_kernels)

    def _device_pointers(self, device):
        if self._device_arrays is not None:
            return [None if t is None else t.data_ptr() for t in self._device_arrays]
        key = str(device)
        if key not in self._dev:
            torch = _torch()
            n = self._n
            parts = [self.q_start, self.kv_start,
                     self.kc_start if self.kc_start is not None else np.zeros(n, np.int64),
                     self.q_len, self.q_pos0, self.kv_len]
            host = np.concatenate([a.view(np.uint8) for a in parts])
            buf = torch.from_numpy(host).to(device)
            base = buf.data_ptr()
            offs = [0, 8 * n, 16 * n, 24 * n, 28 * n, 32 * n]
            ptrs = [base + o for o in offs]
            # order of the C struct: q_start, q_len, q_pos0, kv_start, kv_len, kc_start
            self._dev[key] = (buf, [ptrs[0], ptrs[3], ptrs[4], ptrs[1], ptrs[5],
                                    ptrs[2] if self.kc_start is not None else None])
        return self._dev[key][1]

    def c(self, device=None) -> _CSeqs:
        """The C struct.  With a device: pointers to the device copies (made once per device).
        Without one, host pointers stand in: only the host bounds may then be used (workspace
        sizes, argument checks); no launch may be given such a struct."""
        if device is not None:
            p = self._device_pointers(device)
        elif self._device_arrays is not None:
            p = self._device_pointers(None)
        else:
            kc = self.kc_start
            p = [self.q_start.ctypes.data, self.q_len.ctypes.data, self.q_pos0.ctypes.data,
                 self.kv_start.ctypes.data, self.kv_len.ctypes.data,
                 kc.ctypes.data if kc is not None else None]
        return _CSeqs(self.num_seqs, self.max_q_len, self.max_kv_len, self.q_rows, *p)


def _device_ints(a, device, name):
    """A device int32 array: a device tensor as given, or a host array copied to the device."""
    if a is None:
        return None, None
    torch = _torch()
    if isinstance(a, torch.Tensor):
        if a.device.type != "cuda" or a.dtype != torch.int32 or not a.is_contiguous():
            raise ValueError(f"{name} must be a contiguous int32 device tensor")
        return a, ctypes.c_void_p(a.data_ptr())
    t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.int32)).to(device)
    return t, ctypes.c_void_p(t.data_ptr())


# ----------------------------------------------------------------------------- calls

def _torch():
    import torch
    return torch


def _ptr(t, name, dtype=None, ndim=None):
    torch = _torch()
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.device.type != "cuda":
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if dtype is not None and t.dtype != dtype:
        raise TypeError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if ndim is not None and t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dimensions")
    return ctypes.c_void_p(t.data_ptr())


def _elem_dtype(p: Params):
    torch = _torch()
    return torch.bfloat16 if p.dtype == BF16 else torch.float32


def _stream(stream, device):
    torch = _torch()
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _check(status: int, func: str):
    if status != 0:
        lib = load_library()
        raise InfLLM2Error(status, func, lib.infllm2_last_error().decode())


def compress_kernels(params, seqs: Seqs, k, kernels, prev_kv_len=None, stream=None):
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    keep, prev = _device_ints(prev_kv_len, k.device, "prev_kv_len")
    cp, cs = p.c(), seqs.c(k.device)
    _check(lib.infllm2_compress_kernels(ctypes.byref(cp), ctypes.byref(cs), _ptr(k, "k", dt),
                                        prev, _ptr(kernels, "kernels", dt),
                                        _stream(stream, k.device)),
           "infllm2_compress_kernels")


def block_scores(params, seqs: Seqs, q, kernels, scores, stream=None):
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    torch = _torch()
    cp, cs = p.c(), seqs.c(q.device)
    _check(lib.infllm2_block_scores(ctypes.byref(cp), ctypes.byref(cs), _ptr(q, "q", dt),
                                    _ptr(kernels, "kernels", dt),
                                    _ptr(scores, "scores", torch.float32, 3),
                                    int(scores.shape[2]), _stream(stream, q.device)),
           "infllm2_block_scores")


def topk_select(params, seqs: Seqs, scores, block_idx, stream=None):
    p = Params.from_any(params)
    lib = load_library()
    torch = _torch()
    cp, cs = p.c(), seqs.c(scores.device)
    _check(lib.infllm2_topk_select(ctypes.byref(cp), ctypes.byref(cs),
                                   _ptr(scores, "scores", torch.float32, 3), int(scores.shape[2]),
                                   _ptr(block_idx, "block_idx", torch.int32),
                                   _stream(stream, scores.device)),
           "infllm2_topk_select")


def sparse_attn_prefill(params, seqs: Seqs, q, k, v, block_idx, out, lse=None, stream=None):
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    torch = _torch()
    cp, cs = p.c(), seqs.c(q.device)
    _check(lib.infllm2_sparse_attn_prefill(
        ctypes.byref(cp), ctypes.byref(cs), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(block_idx, "block_idx", torch.int32), _ptr(out, "out", dt),
        _ptr(lse, "lse", torch.float32) if lse is not None else None,
        _stream(stream, q.device)), "infllm2_sparse_attn_prefill")


def decode_workspace_size(params, total_q_rows: int, num_splits: int = 0) -> int:
    p = Params.from_any(params)
    cp = p.c()
    return int(load_library().infllm2_decode_workspace_size(ctypes.byref(cp), int(total_q_rows),
                                                             int(num_splits)))


def sparse_attn_decode(params, seqs: Seqs, q, k, v, block_idx, out, lse=None, num_splits=0,
                       workspace=None, stream=None):
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    torch = _torch()
    cp, cs = p.c(), seqs.c(q.device)
    ws_ptr, ws_bytes = None, 0
    if workspace is not None:
        ws_ptr = _ptr(workspace, "workspace")
        ws_bytes = workspace.numel() * workspace.element_size()
    _check(lib.infllm2_sparse_attn_decode(
        ctypes.byref(cp), ctypes.byref(cs), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(block_idx, "block_idx", torch.int32), int(num_splits), ws_ptr, ws_bytes,
        _ptr(out, "out", dt), _ptr(lse, "lse", torch.float32) if lse is not None else None,
        _stream(stream, q.device)), "infllm2_sparse_attn_decode")


def decode_step_fused(params, seqs: Seqs, q, k_cache, v_cache, kernels, prev_kv_len, scores,
                      block_idx, out, lse, workspace, num_splits=0, stream=None):
    """infllm2_decode_step: the four decode stages in one library call."""
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    torch = _torch()
    keep, prev = _device_ints(prev_kv_len, q.device, "prev_kv_len")
    cp, cs = p.c(), seqs.c(q.device)
    _check(lib.infllm2_decode_step(
        ctypes.byref(cp), ctypes.byref(cs), _ptr(q, "q", dt), _ptr(k_cache, "k_cache", dt),
        _ptr(v_cache, "v_cache", dt), _ptr(kernels, "kernels", dt), prev,
        _ptr(scores, "scores", torch.float32, 3), int(scores.shape[2]),
        _ptr(block_idx, "block_idx", torch.int32), int(num_splits), _ptr(workspace, "workspace"),
        workspace.numel() * workspace.element_size(), _ptr(out, "out", dt),
        _ptr(lse, "lse", torch.float32) if lse is not None else None,
        _stream(stream, q.device)), "infllm2_decode_step")


def decode_step_noalloc(params, seqs: Seqs, q, k_cache, v_cache, kernels, prev_kv_len, scores,
                        block_idx, out, lse, num_splits=0, stream=None):
    """infllm2_decode_step_noalloc: the decode step with the library's own device workspace
    (no workspace argument, nothing allocated by the library)."""
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    torch = _torch()
    keep, prev = _device_ints(prev_kv_len, q.device, "prev_kv_len")
    cp, cs = p.c(), seqs.c(q.device)
    _check(lib.infllm2_decode_step_noalloc(
        ctypes.byref(cp), ctypes.byref(cs), _ptr(q, "q", dt), _ptr(k_cache, "k_cache", dt),
        _ptr(v_cache, "v_cache", dt), _ptr(kernels, "kernels", dt), prev,
        _ptr(scores, "scores", torch.float32, 3), int(scores.shape[2]),
        _ptr(block_idx, "block_idx", torch.int32), int(num_splits), _ptr(out, "out", dt),
        _ptr(lse, "lse", torch.float32) if lse is not None else None,
        _stream(stream, q.device)), "infllm2_decode_step_noalloc")


def backward_workspace_size(params, seqs: Seqs) -> int:
    """Bytes of workspace sparse_attn_backward needs (0: invalid or unsupported arguments)."""
    p = Params.from_any(params)
    cp, cs = p.c(), seqs.c()
    return int(load_library().infllm2_backward_workspace_size(ctypes.byref(cp), ctypes.byref(cs)))


def sparse_attn_backward(params, seqs: Seqs, q, k, v, block_idx, out, lse, dout, dq, dk, dv,
                         workspace, stream=None):
    """infllm2_sparse_attn_backward: float32 dq, dk, dv for the upstream gradient dout."""
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    torch = _torch()
    f32 = torch.float32
    cp, cs = p.c(), seqs.c(q.device)
    _check(lib.infllm2_sparse_attn_backward(
        ctypes.byref(cp), ctypes.byref(cs), _ptr(q, "q", dt), _ptr(k, "k", dt), _ptr(v, "v", dt),
        _ptr(block_idx, "block_idx", torch.int32), _ptr(out, "out", dt), _ptr(lse, "lse", f32),
        _ptr(dout, "dout", dt), _ptr(dq, "dq", f32), _ptr(dk, "dk", f32), _ptr(dv, "dv", f32),
        _ptr(workspace, "workspace"), workspace.numel() * workspace.element_size(),
        _stream(stream, q.device)), "infllm2_sparse_attn_backward")


def sliding_window_attn(params, seqs: Seqs, window: int, q, k, v, out, lse=None, stream=None):
    """infllm2_sliding_window_attn: attention over the last `window` tokens of each query."""
    p = Params.from_any(params)
    lib = load_library()
    dt = _elem_dtype(p)
    torch = _torch()
    cp, cs = p.c(), seqs.c(q.device)
    _check(lib.infllm2_sliding_window_attn(
        ctypes.byref(cp), ctypes.byref(cs), int(window), _ptr(q, "q", dt), _ptr(k, "k", dt),
        _ptr(v, "v", dt), _ptr(out, "out", dt),
        _ptr(lse, "lse", torch.float32) if lse is not None else None,
        _stream(stream, q.device)), "infllm2_sliding_window_attn")
