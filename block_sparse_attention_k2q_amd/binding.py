"""Thin ctypes binding of libmsa.so (include/msa.h).

Every function named ``msa_*`` here mirrors the C entry point of the same name:
it checks dtypes/shapes/devices of torch tensors, passes raw pointers and the
stream, and maps the status to an exception.  All computation happens in the
HIP kernels; PyTorch only provides device memory and streams.

The library is loaded on first use, never at import (msa_bindings page:
``kernels()`` binds lazily; a failed bind is not cached, so a later call
retries).  A missing library raises ``UnavailableError``.
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
import threading
from typing import Optional

import numpy as np
import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libmsa.so")

(MSA_OK, MSA_ERR_INVALID, MSA_ERR_UNSUPPORTED, MSA_ERR_SHAPE, MSA_ERR_ALIGN, MSA_ERR_HIP,
 MSA_ERR_SCRATCH_LIMIT) = range(7)
NOALLOC_SCRATCH_BYTES = 64 << 20   # MSA_NOALLOC_SCRATCH_BYTES (msa.h)
SCHED_ERR_DROPPED, SCHED_ERR_GEOMETRY = 0, 1
DQ_RECOMPUTE, DQ_ATOMIC_POOL, DQ_DS_BUFFER, DQ_ATOMIC_POOL_BF16 = 0, 1, 2, 3
MAX_DOC_CHUNKS = 1 << 18
INDEX_DIM = 128                  # MSA_INDEX_DIM (msa.h)
INDEX_MAX_DOC_BLOCKS = 4096      # MSA_INDEX_MAX_DOC_BLOCKS (msa.h)

EXPORTED = (
    "msa_device_check", "msa_schedule_layout_of", "msa_build_schedule", "msa_forward",
    "msa_backward_scratch_bytes", "msa_backward", "msa_backward_preprocess", "msa_backward_main",
    "msa_backward_dq", "msa_backward_postprocess", "msa_grid_launch_bound", "msa_status_string",
    "msa_index_scratch_bytes", "msa_index_select", "msa_backward_noalloc", "msa_build_schedule_kv",
    "msa_forward_kv_scratch_bytes", "msa_forward_kv",
)


class UnavailableError(RuntimeError):
    """libmsa.so is missing or cannot be loaded on this host."""


class MSAProblem(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int32) for n in (
        "total_tokens", "num_docs", "num_kv_heads", "q_per_kv", "head_dim", "block_size",
        "query_chunk", "topk", "num_chunks", "num_kblocks", "max_doc_chunks", "num_cus")] + [
        ("softmax_scale", ctypes.c_float), ("dq_mode", ctypes.c_int32), ("kv_rows", ctypes.c_int32)]


class MSAScheduleLayout(ctypes.Structure):
    _fields_ = [(n, ctypes.c_int64) for n in (
        "desc", "err", "doc_chunk_off", "doc_blk_off", "doc_kv_off", "chunk_doc", "sel_clean", "row_cursor",
        "row_ptr", "head_off", "q_idx", "task_meta", "total")]


_lib = None
_lib_lock = threading.Lock()


def lib() -> ctypes.CDLL:
    """Load libmsa.so once per process; a failure is not cached."""
    global _lib
    if _lib is not None:
        return _lib
    with _lib_lock:
        if _lib is not None:
            return _lib
        if not os.path.exists(LIB_PATH):
            raise UnavailableError(
                f"{LIB_PATH} is not built; run `python -m block_sparse_attention_k2q_amd.build`")
        try:
            h = ctypes.CDLL(LIB_PATH)
        except OSError as e:
            raise UnavailableError(f"cannot load {LIB_PATH}: {e}") from e
        P = ctypes.POINTER(MSAProblem)
        vp, i32p = ctypes.c_void_p, ctypes.c_void_p
        sig = {
            "msa_device_check": ([ctypes.c_int, ctypes.POINTER(ctypes.c_int32)], ctypes.c_int),
            "msa_schedule_layout_of": ([P, ctypes.POINTER(MSAScheduleLayout)], ctypes.c_int),
            "msa_build_schedule": ([P, i32p, i32p, i32p, vp], ctypes.c_int),
            "msa_build_schedule_kv": ([P, i32p, i32p, i32p, i32p, vp], ctypes.c_int),
            "msa_forward": ([P, vp, vp, vp, i32p, i32p, vp, vp, vp], ctypes.c_int),
            "msa_forward_kv_scratch_bytes": ([P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
            "msa_forward_kv": ([P, vp, vp, vp, i32p, i32p, vp, vp, vp, vp], ctypes.c_int),
            "msa_backward_scratch_bytes": ([P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
            "msa_backward": ([P, vp, vp, vp, vp, vp, vp, i32p, i32p, vp, vp, vp, vp, vp], ctypes.c_int),
            "msa_backward_preprocess": ([P, vp, vp, vp, vp], ctypes.c_int),
            "msa_backward_main": ([P, vp, vp, vp, vp, vp, i32p, i32p, vp, vp], ctypes.c_int),
            "msa_backward_dq": ([P, vp, vp, vp, vp, vp, i32p, i32p, vp, vp, vp], ctypes.c_int),
            "msa_backward_postprocess": ([P, i32p, vp, vp, vp, vp, vp], ctypes.c_int),
            "msa_grid_launch_bound": ([ctypes.c_int64, ctypes.c_int32], ctypes.c_int64),
            "msa_status_string": ([ctypes.c_int], ctypes.c_char_p),
            "msa_index_scratch_bytes": ([P, ctypes.POINTER(ctypes.c_size_t)], ctypes.c_int),
            "msa_index_select": ([P, vp, vp, i32p, vp, i32p, vp], ctypes.c_int),
            "msa_backward_noalloc": ([P, vp, vp, vp, vp, vp, vp, i32p, i32p, vp, vp, vp, vp], ctypes.c_int),
        }
        for name, (args, res) in sig.items():
            fn = getattr(h, name)
            fn.argtypes = args
            fn.restype = res
        _lib = h
        return h


def _check(status: int, what: str) -> None:
    if status == MSA_OK:
        return
    msg = f"{what}: {lib().msa_status_string(status).decode()}"
    if status == MSA_ERR_UNSUPPORTED:
        raise NotImplementedError(msg)
    if status in (MSA_ERR_INVALID, MSA_ERR_SHAPE, MSA_ERR_ALIGN, MSA_ERR_SCRATCH_LIMIT):
        raise ValueError(msg)
    raise RuntimeError(msg)


_cus_cache: dict[int, int] = {}


def msa_device_check(device: int = 0) -> int:
    """Raise NotImplementedError unless `device` is gfx950; return its CU count (memoised)."""
    if device in _cus_cache:
        return _cus_cache[device]
    n = ctypes.c_int32(0)
    _check(lib().msa_device_check(int(device), ctypes.byref(n)), f"device {device}")
    _cus_cache[device] = int(n.value)
    return _cus_cache[device]


# ---------------------------------------------------------------------------
# Problem description (host integers computed from the host copy of cu_seqlens)
# ---------------------------------------------------------------------------

@dataclasses.dataclass(frozen=True)
class Problem:
    total_tokens: int
    num_docs: int
    num_kv_heads: int
    head_dim: int
    topk: int
    num_chunks: int
    num_kblocks: int
    max_doc_chunks: int
    num_cus: int
    softmax_scale: float
    q_per_kv: int = 16
    block_size: int = 64
    query_chunk: int = 8
    dq_mode: int = DQ_DS_BUFFER
    kv_rows: int = 0           # rows of k, v, dk, dv; 0 = total_tokens (compact)

    @staticmethod
    def make(cu_seqlens, num_kv_heads: int, head_dim: int, topk: int, num_cus: int = 256,
             softmax_scale: Optional[float] = None, block_size: int = 64,
             dq_mode: int = DQ_DS_BUFFER, kv_rows: int = 0) -> "Problem":
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        lens = np.diff(cu)
        nch = -(-lens // 8)
        return Problem(total_tokens=int(cu[-1]), num_docs=len(lens), num_kv_heads=int(num_kv_heads),
                       head_dim=int(head_dim), topk=int(topk), num_chunks=int(nch.sum()),
                       num_kblocks=int((-(-lens // block_size)).sum()),
                       max_doc_chunks=int(nch.max(initial=0)), num_cus=int(num_cus),
                       softmax_scale=float(head_dim ** -0.5 if softmax_scale is None else softmax_scale),
                       block_size=int(block_size), dq_mode=int(dq_mode), kv_rows=int(kv_rows))

    @property
    def num_q_heads(self) -> int:
        return self.num_kv_heads * self.q_per_kv

    @property
    def kv_total(self) -> int:
        """Rows of k, v, dk, dv."""
        return self.kv_rows if self.kv_rows > 0 else self.total_tokens

    @property
    def capacity(self) -> int:
        return self.num_kv_heads * self.num_chunks * self.topk

    def c_struct(self) -> MSAProblem:
        return MSAProblem(self.total_tokens, self.num_docs, self.num_kv_heads, self.q_per_kv,
                          self.head_dim, self.block_size, self.query_chunk, self.topk,
                          self.num_chunks, self.num_kblocks, self.max_doc_chunks, self.num_cus,
                          self.softmax_scale, self.dq_mode, self.kv_rows)


def _ptr(t: Optional[torch.Tensor]) -> Optional[int]:
    return None if t is None else t.data_ptr()


def _stream(stream) -> Optional[int]:
    if stream is None:
        return torch.cuda.current_stream().cuda_stream
    return getattr(stream, "cuda_stream", stream)


def _on_device(*tensors):
    """The tensors' one GPU, made current for the call (the library launches on
    the current device, on that device's current stream unless one is given)."""
    devs = {t.device for t in tensors if t is not None}
    if len(devs) != 1:
        raise ValueError(f"all tensors must be on one GPU, got {sorted(str(d) for d in devs)}")
    return torch.cuda.device(next(iter(devs)))


def _expect(t: torch.Tensor, name: str, dtype: torch.dtype, shape: tuple) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a device tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def msa_schedule_layout_of(p: Problem) -> MSAScheduleLayout:
    out = MSAScheduleLayout()
    ps = p.c_struct()
    _check(lib().msa_schedule_layout_of(ctypes.byref(ps), ctypes.byref(out)), "schedule layout")
    return out


def msa_build_schedule(p: Problem, cu_seqlens: torch.Tensor, sel: torch.Tensor, sched: torch.Tensor,
                       stream=None) -> None:
    L = msa_schedule_layout_of(p)
    _expect(cu_seqlens, "cu_seqlens", torch.int32, (p.num_docs + 1,))
    _expect(sel, "sel", torch.int32, (p.num_kv_heads, p.num_chunks, p.topk))
    _expect(sched, "sched", torch.int32, (L.total,))
    with _on_device(cu_seqlens, sel, sched):
        ps = p.c_struct()
        _check(lib().msa_build_schedule(ctypes.byref(ps), _ptr(cu_seqlens), _ptr(sel), _ptr(sched),
                                        _stream(stream)), "msa_build_schedule")


def msa_build_schedule_kv(p: Problem, cu_seqlens: torch.Tensor, sel: torch.Tensor,
                          kv_starts: Optional[torch.Tensor], sched: torch.Tensor, stream=None) -> None:
    """msa_build_schedule with each document's keys at row kv_starts[d] of
    k / v (int32 [num_docs] on the device; None = the cu_seqlens rows)."""
    L = msa_schedule_layout_of(p)
    _expect(cu_seqlens, "cu_seqlens", torch.int32, (p.num_docs + 1,))
    _expect(sel, "sel", torch.int32, (p.num_kv_heads, p.num_chunks, p.topk))
    _expect(sched, "sched", torch.int32, (L.total,))
    if kv_starts is not None:
        _expect(kv_starts, "kv_starts", torch.int32, (p.num_docs,))
    with _on_device(cu_seqlens, sel, sched, kv_starts):
        ps = p.c_struct()
        _check(lib().msa_build_schedule_kv(ctypes.byref(ps), _ptr(cu_seqlens), _ptr(sel), _ptr(kv_starts),
                                           _ptr(sched), _stream(stream)), "msa_build_schedule_kv")


def msa_forward(p: Problem, q, k, v, cu_seqlens, sched, out, lse, stream=None) -> None:
    T, hq, hkv, D, W = p.total_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim, p.kv_total
    for name, t, shape in (("q", q, (T, hq, D)), ("k", k, (W, hkv, D)), ("v", v, (W, hkv, D)),
                           ("out", out, (T, hq, D))):
        _expect(t, name, torch.bfloat16, shape)
    _expect(lse, "lse", torch.float32, (T, hq))
    _expect(cu_seqlens, "cu_seqlens", torch.int32, (p.num_docs + 1,))
    _expect(sched, "sched", torch.int32, (msa_schedule_layout_of(p).total,))
    with _on_device(q, k, v, cu_seqlens, sched, out, lse):
        ps = p.c_struct()
        _check(lib().msa_forward(ctypes.byref(ps), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(sched),
                                 _ptr(out), _ptr(lse), _stream(stream)), "msa_forward")


def msa_forward_kv_scratch_bytes(p: Problem) -> int:
    ps = p.c_struct()
    out = ctypes.c_size_t(0)
    _check(lib().msa_forward_kv_scratch_bytes(ctypes.byref(ps), ctypes.byref(out)), "msa_forward_kv_scratch_bytes")
    return int(out.value)


def msa_forward_kv(p: Problem, q, k, v, cu_seqlens, sched, scratch, out, lse, stream=None) -> None:
    """Planner-driven forward (KV-parallel over the task table): same out / lse as msa_forward."""
    T, hq, hkv, D, W = p.total_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim, p.kv_total
    for name, t, shape in (("q", q, (T, hq, D)), ("k", k, (W, hkv, D)), ("v", v, (W, hkv, D)),
                           ("out", out, (T, hq, D))):
        _expect(t, name, torch.bfloat16, shape)
    _expect(lse, "lse", torch.float32, (T, hq))
    _expect(cu_seqlens, "cu_seqlens", torch.int32, (p.num_docs + 1,))
    _expect(sched, "sched", torch.int32, (msa_schedule_layout_of(p).total,))
    _expect(scratch, "scratch", torch.uint8, (msa_forward_kv_scratch_bytes(p),))
    with _on_device(q, k, v, cu_seqlens, sched, scratch, out, lse):
        ps = p.c_struct()
        _check(lib().msa_forward_kv(ctypes.byref(ps), _ptr(q), _ptr(k), _ptr(v), _ptr(cu_seqlens), _ptr(sched),
                                    _ptr(scratch), _ptr(out), _ptr(lse), _stream(stream)), "msa_forward_kv")


def forward_kv(p: Problem, q, k, v, cu_seqlens, sched, scratch=None, stream=None):
    if scratch is None:
        scratch = torch.empty(msa_forward_kv_scratch_bytes(p), dtype=torch.uint8, device=q.device)
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    msa_forward_kv(p, q, k, v, cu_seqlens, sched, scratch, out, lse, stream)
    return out, lse


def msa_index_scratch_bytes(p: Problem) -> int:
    ps = p.c_struct()
    out = ctypes.c_size_t(0)
    _check(lib().msa_index_scratch_bytes(ctypes.byref(ps), ctypes.byref(out)), "msa_index_scratch_bytes")
    return int(out.value)


def msa_index_select(p: Problem, qi, ki, cu_seqlens, scratch, sel, stream=None) -> None:
    """Index scorer + top-k block selection into sel int32 [Hkv, C, topk]."""
    T, hkv = p.total_tokens, p.num_kv_heads
    _expect(qi, "qi", torch.bfloat16, (T, hkv, INDEX_DIM))
    _expect(ki, "ki", torch.bfloat16, (T, hkv, INDEX_DIM))
    _expect(cu_seqlens, "cu_seqlens", torch.int32, (p.num_docs + 1,))
    _expect(scratch, "scratch", torch.uint8, (msa_index_scratch_bytes(p),))
    _expect(sel, "sel", torch.int32, (hkv, p.num_chunks, p.topk))
    with _on_device(qi, ki, cu_seqlens, scratch, sel):
        ps = p.c_struct()
        _check(lib().msa_index_select(ctypes.byref(ps), _ptr(qi), _ptr(ki), _ptr(cu_seqlens), _ptr(scratch),
                                      _ptr(sel), _stream(stream)), "msa_index_select")


def index_select(p: Problem, qi, ki, cu_seqlens, scratch=None, stream=None) -> torch.Tensor:
    if scratch is None:
        scratch = torch.empty(msa_index_scratch_bytes(p), dtype=torch.uint8, device=qi.device)
    sel = torch.empty(p.num_kv_heads, p.num_chunks, p.topk, dtype=torch.int32, device=qi.device)
    msa_index_select(p, qi, ki, cu_seqlens, scratch, sel, stream)
    return sel


def msa_backward_scratch_bytes(p: Problem) -> int:
    n = ctypes.c_size_t(0)
    ps = p.c_struct()
    _check(lib().msa_backward_scratch_bytes(ctypes.byref(ps), ctypes.byref(n)), "scratch size")
    return int(n.value)


def _check_bwd_inputs(p: Problem, q, k, v, out, dout, lse, cu_seqlens, sched, scratch):
    T, hq, hkv, D, W = p.total_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim, p.kv_total
    for name, t, shape in (("q", q, (T, hq, D)), ("k", k, (W, hkv, D)), ("v", v, (W, hkv, D)),
                           ("out", out, (T, hq, D)), ("dout", dout, (T, hq, D))):
        if t is not None:
            _expect(t, name, torch.bfloat16, shape)
    if lse is not None:
        _expect(lse, "lse", torch.float32, (T, hq))
    if cu_seqlens is not None:
        _expect(cu_seqlens, "cu_seqlens", torch.int32, (p.num_docs + 1,))
    if sched is not None:
        _expect(sched, "sched", torch.int32, (msa_schedule_layout_of(p).total,))
    if scratch is not None:
        _expect(scratch, "scratch", torch.uint8, (msa_backward_scratch_bytes(p),))


def msa_backward(p: Problem, q, k, v, out, dout, lse, cu_seqlens, sched, scratch, dq, dk, dv,
                 stream=None) -> None:
    _check_bwd_inputs(p, q, k, v, out, dout, lse, cu_seqlens, sched, scratch)
    T, hq, hkv, D = p.total_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim
    _expect(dq, "dq", torch.bfloat16, (T, hq, D))
    _expect(dk, "dk", torch.bfloat16, (p.kv_total, hkv, D))
    _expect(dv, "dv", torch.bfloat16, (p.kv_total, hkv, D))
    with _on_device(q, k, v, out, dout, lse, cu_seqlens, sched, scratch, dq, dk, dv):
        ps = p.c_struct()
        _check(lib().msa_backward(ctypes.byref(ps), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                  _ptr(lse), _ptr(cu_seqlens), _ptr(sched), _ptr(scratch), _ptr(dq),
                                  _ptr(dk), _ptr(dv), _stream(stream)), "msa_backward")


def msa_backward_noalloc(p: Problem, q, k, v, out, dout, lse, cu_seqlens, sched, dq, dk, dv,
                         stream=None) -> None:
    """msa_backward with the library's static scratch (allocates nothing;
    ValueError when the problem needs more than NOALLOC_SCRATCH_BYTES)."""
    _check_bwd_inputs(p, q, k, v, out, dout, lse, cu_seqlens, sched, None)
    T, hq, hkv, D = p.total_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim
    _expect(dq, "dq", torch.bfloat16, (T, hq, D))
    _expect(dk, "dk", torch.bfloat16, (p.kv_total, hkv, D))
    _expect(dv, "dv", torch.bfloat16, (p.kv_total, hkv, D))
    with _on_device(q, k, v, out, dout, lse, cu_seqlens, sched, dq, dk, dv):
        ps = p.c_struct()
        _check(lib().msa_backward_noalloc(ctypes.byref(ps), _ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout),
                                          _ptr(lse), _ptr(cu_seqlens), _ptr(sched), _ptr(dq), _ptr(dk),
                                          _ptr(dv), _stream(stream)), "msa_backward_noalloc")


def msa_backward_preprocess(p: Problem, out, dout, scratch, stream=None) -> None:
    _check_bwd_inputs(p, None, None, None, out, dout, None, None, None, scratch)
    with _on_device(out, dout, scratch):
        ps = p.c_struct()
        _check(lib().msa_backward_preprocess(ctypes.byref(ps), _ptr(out), _ptr(dout), _ptr(scratch),
                                             _stream(stream)), "msa_backward_preprocess")


def msa_backward_main(p: Problem, q, k, v, dout, lse, cu_seqlens, sched, scratch, stream=None) -> None:
    _check_bwd_inputs(p, q, k, v, None, dout, lse, cu_seqlens, sched, scratch)
    with _on_device(q, k, v, dout, lse, cu_seqlens, sched, scratch):
        ps = p.c_struct()
        _check(lib().msa_backward_main(ctypes.byref(ps), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                       _ptr(cu_seqlens), _ptr(sched), _ptr(scratch), _stream(stream)),
               "msa_backward_main")


def msa_backward_dq(p: Problem, q, k, v, dout, lse, cu_seqlens, sched, scratch, dq, stream=None) -> None:
    _check_bwd_inputs(p, q, k, v, None, dout, lse, cu_seqlens, sched, scratch)
    T, hq, D = p.total_tokens, p.num_q_heads, p.head_dim
    _expect(dq, "dq", torch.bfloat16, (T, hq, D))
    with _on_device(q, k, v, dout, lse, cu_seqlens, sched, scratch, dq):
        ps = p.c_struct()
        _check(lib().msa_backward_dq(ctypes.byref(ps), _ptr(q), _ptr(k), _ptr(v), _ptr(dout), _ptr(lse),
                                     _ptr(cu_seqlens), _ptr(sched), _ptr(scratch), _ptr(dq), _stream(stream)),
               "msa_backward_dq")


def msa_backward_postprocess(p: Problem, sched, scratch, dq, dk, dv, stream=None) -> None:
    _check_bwd_inputs(p, None, None, None, None, None, None, None, sched, scratch)
    T, hq, hkv, D = p.total_tokens, p.num_q_heads, p.num_kv_heads, p.head_dim
    _expect(dq, "dq", torch.bfloat16, (T, hq, D))
    _expect(dk, "dk", torch.bfloat16, (p.kv_total, hkv, D))
    _expect(dv, "dv", torch.bfloat16, (p.kv_total, hkv, D))
    with _on_device(sched, scratch, dq, dk, dv):
        ps = p.c_struct()
        _check(lib().msa_backward_postprocess(ctypes.byref(ps), _ptr(sched), _ptr(scratch), _ptr(dq), _ptr(dk),
                                              _ptr(dv), _stream(stream)), "msa_backward_postprocess")


def msa_grid_launch_bound(capacity: int, num_cus: int) -> int:
    return int(lib().msa_grid_launch_bound(int(capacity), int(num_cus)))


# ---------------------------------------------------------------------------
# Allocation helpers (torch owns the memory) and schedule views
# ---------------------------------------------------------------------------

def alloc_schedule(p: Problem, device="cuda") -> torch.Tensor:
    return torch.empty(msa_schedule_layout_of(p).total, dtype=torch.int32, device=device)


def alloc_scratch(p: Problem, device="cuda") -> torch.Tensor:
    return torch.empty(msa_backward_scratch_bytes(p), dtype=torch.uint8, device=device)


def schedule_views(p: Problem, sched: torch.Tensor) -> dict:
    """Named views into a schedule workspace (no copies)."""
    L = msa_schedule_layout_of(p)
    hkv, C, K, R = p.num_kv_heads, p.num_chunks, p.topk, p.num_kblocks
    cap = hkv * C * K
    return dict(
        desc=sched[L.desc:L.desc + 8], err=sched[L.err:L.err + 8],
        doc_chunk_off=sched[L.doc_chunk_off:L.doc_chunk_off + p.num_docs + 1],
        doc_blk_off=sched[L.doc_blk_off:L.doc_blk_off + p.num_docs + 1],
        doc_kv_off=sched[L.doc_kv_off:L.doc_kv_off + p.num_docs],
        chunk_doc=sched[L.chunk_doc:L.chunk_doc + C],
        sel_clean=sched[L.sel_clean:L.sel_clean + cap].view(hkv, C, K),
        row_ptr=sched[L.row_ptr:L.row_ptr + hkv * (R + 1)].view(hkv, R + 1),
        head_off=sched[L.head_off:L.head_off + hkv + 1],
        q_idx=sched[L.q_idx:L.q_idx + cap].view(hkv, C * K),
        task_meta=sched[L.task_meta:L.task_meta + cap * 6].view(cap, 6),
    )


def build_schedule(p: Problem, cu_seqlens: torch.Tensor, sel: torch.Tensor, stream=None) -> torch.Tensor:
    sched = alloc_schedule(p, cu_seqlens.device)
    msa_build_schedule(p, cu_seqlens, sel, sched, stream)
    return sched


def forward(p: Problem, q, k, v, cu_seqlens, sched, stream=None):
    out = torch.empty_like(q)
    lse = torch.empty(q.shape[0], q.shape[1], dtype=torch.float32, device=q.device)
    msa_forward(p, q, k, v, cu_seqlens, sched, out, lse, stream)
    return out, lse


def backward(p: Problem, q, k, v, out, dout, lse, cu_seqlens, sched, scratch=None, stream=None):
    if scratch is None:
        scratch = alloc_scratch(p, q.device)
    dq = torch.empty_like(q)
    dk = torch.empty_like(k)
    dv = torch.empty_like(v)
    msa_backward(p, q, k, v, out, dout, lse, cu_seqlens, sched, scratch, dq, dk, dv, stream)
    return dq, dk, dv
