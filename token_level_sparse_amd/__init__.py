"""Python binding of libtokenselect.so (the gfx950 decode-step path).

Argument marshalling only: every step of the path runs in the HIP kernels behind
the C ABI of include/tokenselect.h. The functions below carry the same names as
the C entry points without the ``tokenselect_`` prefix, take torch tensors that
already live on the GPU (PyTorch is used for device memory and streams), and
raise ``TokenSelectError`` on a non-OK status. There is no fallback: if the
library is not built, loading it raises.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Optional

import torch

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libtokenselect.so")

TS_OK, TS_ERR_INVALID_ARG, TS_ERR_UNSUPPORTED, TS_ERR_WORKSPACE, TS_ERR_DEVICE = range(5)
TS_F32, TS_BF16 = 0, 1

ENTRY_POINTS = (
    "tokenselect_workspace_size",
    "tokenselect_score",
    "tokenselect_vote_topk",
    "tokenselect_sparse_attn",
    "tokenselect_decode_step",
    "tokenselect_decode_step_noalloc",
    "tokenselect_prefill_workspace_size",
    "tokenselect_prefill_select",
    "tokenselect_chunk_attn",
    "tokenselect_prefill_chunk",
    "tokenselect_ablation_workspace_size",
    "tokenselect_select_ablation",
    "tokenselect_validate",
    "tokenselect_validate_selection",
    "tokenselect_status_string",
    "tokenselect_last_error",
)


class TokenSelectError(RuntimeError):
    def __init__(self, status: int, message: str):
        super().__init__(f"status {status}: {message}")
        self.status = status


class Shape(ctypes.Structure):
    _fields_ = [
        ("num_q_heads", ctypes.c_int32),
        ("num_kv_heads", ctypes.c_int32),
        ("head_dim", ctypes.c_int32),
        ("page_size", ctypes.c_int32),
        ("batch", ctypes.c_int32),
        ("block_table_stride", ctypes.c_int32),
        ("max_total_tokens", ctypes.c_int64),
        ("dtype", ctypes.c_int32),
    ]


class Select(ctypes.Structure):
    _fields_ = [
        ("top_k", ctypes.c_int32),
        ("n_local", ctypes.c_int32),
        ("score_scale", ctypes.c_float),
        ("attn_scale", ctypes.c_float),
        ("cos_threshold", ctypes.c_double),
        ("top_p", ctypes.c_double),
    ]


class Cache(ctypes.Structure):
    _fields_ = [
        ("cached_q", ctypes.c_void_p),
        ("cached_idx", ctypes.c_void_p),
        ("cached_count", ctypes.c_void_p),
        ("valid", ctypes.c_void_p),
    ]


_lib_handle = None


def load_library(path: Optional[str] = None) -> ctypes.CDLL:
    """Load the built library (once). Raises if it is missing."""
    global _lib_handle
    if _lib_handle is not None and path is None:
        return _lib_handle
    p = path or LIB_PATH
    if not os.path.exists(p):
        raise RuntimeError(f"{p} is not built; run token_level_sparse_amd.build.build()")
    lib = ctypes.CDLL(p)
    vp, sz = ctypes.c_void_p, ctypes.c_size_t
    sp, selp = ctypes.POINTER(Shape), ctypes.POINTER(Select)
    lib.tokenselect_workspace_size.argtypes = [sp, selp]
    lib.tokenselect_workspace_size.restype = sz
    lib.tokenselect_score.argtypes = [sp, selp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tokenselect_score.restype = ctypes.c_int
    lib.tokenselect_vote_topk.argtypes = [sp, selp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tokenselect_vote_topk.restype = ctypes.c_int
    lib.tokenselect_sparse_attn.argtypes = [sp, selp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tokenselect_sparse_attn.restype = ctypes.c_int
    lib.tokenselect_decode_step.argtypes = [sp, selp, vp, vp, vp, vp, vp, ctypes.POINTER(Cache),
                                            vp, vp, vp, sz, vp]
    lib.tokenselect_decode_step.restype = ctypes.c_int
    lib.tokenselect_decode_step_noalloc.argtypes = [sp, selp, vp, vp, vp, vp, vp, ctypes.POINTER(Cache),
                                                    vp, vp, vp]
    lib.tokenselect_decode_step_noalloc.restype = ctypes.c_int
    i32 = ctypes.c_int32
    lib.tokenselect_prefill_workspace_size.argtypes = [sp, selp, i32]
    lib.tokenselect_prefill_workspace_size.restype = sz
    lib.tokenselect_prefill_select.argtypes = [sp, selp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                               vp, sz, vp]
    lib.tokenselect_prefill_select.restype = ctypes.c_int
    lib.tokenselect_chunk_attn.argtypes = [sp, selp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tokenselect_chunk_attn.restype = ctypes.c_int
    lib.tokenselect_prefill_chunk.argtypes = [sp, selp, i32, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              sz, vp]
    lib.tokenselect_prefill_chunk.restype = ctypes.c_int
    lib.tokenselect_ablation_workspace_size.argtypes = [sp, selp, i32, i32]
    lib.tokenselect_ablation_workspace_size.restype = sz
    lib.tokenselect_select_ablation.argtypes = [sp, selp, i32, i32, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    lib.tokenselect_select_ablation.restype = ctypes.c_int
    lib.tokenselect_validate.argtypes = [sp, vp, vp, ctypes.c_int64, vp, vp]
    lib.tokenselect_validate.restype = ctypes.c_int
    lib.tokenselect_validate_selection.argtypes = [sp, selp, vp, vp, vp, vp, vp]
    lib.tokenselect_validate_selection.restype = ctypes.c_int
    lib.tokenselect_status_string.argtypes = [ctypes.c_int]
    lib.tokenselect_status_string.restype = ctypes.c_char_p
    lib.tokenselect_last_error.argtypes = []
    lib.tokenselect_last_error.restype = ctypes.c_char_p
    if path is None:
        _lib_handle = lib
    return lib


def _check(status: int) -> None:
    if status != TS_OK:
        lib = load_library()
        raise TokenSelectError(status, lib.tokenselect_last_error().decode())


def _ptr(t: Optional[torch.Tensor]):
    if t is None:
        return None
    if not t.is_cuda:
        raise ValueError("tensors passed to the HIP path must live on the GPU")
    if not t.is_contiguous():
        raise ValueError("tensors passed to the HIP path must be contiguous")
    return ctypes.c_void_p(t.data_ptr())


def _stream(stream) -> ctypes.c_void_p:
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def make_shape(num_q_heads, num_kv_heads, batch, block_table_stride, max_total_tokens,
               dtype, head_dim=128, page_size=16) -> Shape:
    dt = dtype if isinstance(dtype, int) else (TS_BF16 if dtype == torch.bfloat16 else TS_F32)
    return Shape(num_q_heads, num_kv_heads, head_dim, page_size, batch, block_table_stride,
                 max_total_tokens, dt)


def make_select(top_k, n_local, score_scale=1.0, attn_scale=1.0 / 128 ** 0.5,
                cos_threshold=0.9, top_p=0.0) -> Select:
    return Select(top_k, n_local, score_scale, attn_scale, cos_threshold, top_p)


def workspace_size(shape: Shape, sel: Select) -> int:
    return int(load_library().tokenselect_workspace_size(ctypes.byref(shape), ctypes.byref(sel)))


def alloc_workspace(shape: Shape, sel: Select, device="cuda") -> torch.Tensor:
    n = workspace_size(shape, sel)
    if n == 0:
        raise TokenSelectError(TS_ERR_INVALID_ARG, load_library().tokenselect_last_error().decode())
    return torch.empty(n, dtype=torch.uint8, device=device)


def score(shape, sel, q, k_pool, block_table, seq_lens, logits, head_stats, ws, stream=None):
    lib = load_library()
    _check(lib.tokenselect_score(ctypes.byref(shape), ctypes.byref(sel), _ptr(q), _ptr(k_pool),
                                 _ptr(block_table), _ptr(seq_lens), _ptr(logits), _ptr(head_stats),
                                 _ptr(ws), ws.numel(), _stream(stream)))


def vote_topk(shape, sel, logits, head_stats, seq_lens, vote, sel_idx, sel_count, ws, stream=None):
    lib = load_library()
    _check(lib.tokenselect_vote_topk(ctypes.byref(shape), ctypes.byref(sel), _ptr(logits),
                                     _ptr(head_stats), _ptr(seq_lens), _ptr(vote), _ptr(sel_idx),
                                     _ptr(sel_count), _ptr(ws), ws.numel(), _stream(stream)))


def sparse_attn(shape, sel, q, k_pool, v_pool, block_table, seq_lens, sel_idx, sel_count, out, ws,
                stream=None):
    lib = load_library()
    _check(lib.tokenselect_sparse_attn(ctypes.byref(shape), ctypes.byref(sel), _ptr(q),
                                       _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                       _ptr(seq_lens), _ptr(sel_idx), _ptr(sel_count), _ptr(out),
                                       _ptr(ws), ws.numel(), _stream(stream)))


@dataclass
class CacheState:
    """Caller-owned Selection Cache buffers (C_Q, C_T, counts, valid flags)."""

    cached_q: torch.Tensor
    cached_idx: torch.Tensor
    cached_count: torch.Tensor
    valid: torch.Tensor

    @staticmethod
    def allocate(batch, num_q_heads, head_dim, top_k, dtype, device="cuda") -> "CacheState":
        return CacheState(
            cached_q=torch.zeros(batch, num_q_heads * head_dim, dtype=dtype, device=device),
            cached_idx=torch.zeros(batch, top_k, dtype=torch.int32, device=device),
            cached_count=torch.zeros(batch, dtype=torch.int32, device=device),
            valid=torch.zeros(batch, dtype=torch.int32, device=device),
        )

    def c_struct(self) -> Cache:
        return Cache(_ptr(self.cached_q), _ptr(self.cached_idx), _ptr(self.cached_count),
                     _ptr(self.valid))


def decode_step(shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache: CacheState, hit, out,
                ws, stream=None):
    lib = load_library()
    cs = cache.c_struct()
    _check(lib.tokenselect_decode_step(ctypes.byref(shape), ctypes.byref(sel), _ptr(q),
                                       _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                       _ptr(seq_lens), ctypes.byref(cs), _ptr(hit), _ptr(out),
                                       _ptr(ws), ws.numel(), _stream(stream)))


# Bytes of the static scratch behind decode_step_noalloc (TS_NOALLOC_SCRATCH_BYTES).
NOALLOC_SCRATCH_BYTES = 64 << 20


def decode_step_noalloc(shape, sel, q, k_pool, v_pool, block_table, seq_lens, cache: CacheState, hit,
                        out, stream=None):
    """tokenselect_decode_step_noalloc: the decode step on the library's static scratch."""
    lib = load_library()
    cs = cache.c_struct()
    _check(lib.tokenselect_decode_step_noalloc(ctypes.byref(shape), ctypes.byref(sel), _ptr(q),
                                               _ptr(k_pool), _ptr(v_pool), _ptr(block_table),
                                               _ptr(seq_lens), ctypes.byref(cs), _ptr(hit), _ptr(out),
                                               _stream(stream)))


# ---------------------------------------------------------------- chunk-wise prefill
def prefill_workspace_size(shape: Shape, sel: Select, max_chunk: int) -> int:
    return int(load_library().tokenselect_prefill_workspace_size(ctypes.byref(shape), ctypes.byref(sel),
                                                                 int(max_chunk)))


def alloc_prefill_workspace(shape: Shape, sel: Select, max_chunk: int, device="cuda") -> torch.Tensor:
    n = prefill_workspace_size(shape, sel, max_chunk)
    if n == 0:
        raise TokenSelectError(TS_ERR_INVALID_ARG, load_library().tokenselect_last_error().decode())
    return torch.empty(n, dtype=torch.uint8, device=device)


def prefill_select(shape, sel, max_chunk, q_chunk, chunk_lens, k_pool, block_table, seq_lens,
                   logits, head_stats, vote, sel_idx, sel_count, ws, stream=None):
    lib = load_library()
    _check(lib.tokenselect_prefill_select(ctypes.byref(shape), ctypes.byref(sel), int(max_chunk),
                                          _ptr(q_chunk), _ptr(chunk_lens), _ptr(k_pool),
                                          _ptr(block_table), _ptr(seq_lens), _ptr(logits),
                                          _ptr(head_stats), _ptr(vote), _ptr(sel_idx),
                                          _ptr(sel_count), _ptr(ws), ws.numel(), _stream(stream)))


def chunk_attn(shape, sel, max_chunk, q_chunk, chunk_lens, k_pool, v_pool, block_table, seq_lens,
               sel_idx, sel_count, out, ws, stream=None):
    lib = load_library()
    _check(lib.tokenselect_chunk_attn(ctypes.byref(shape), ctypes.byref(sel), int(max_chunk),
                                      _ptr(q_chunk), _ptr(chunk_lens), _ptr(k_pool), _ptr(v_pool),
                                      _ptr(block_table), _ptr(seq_lens), _ptr(sel_idx),
                                      _ptr(sel_count), _ptr(out), _ptr(ws), ws.numel(),
                                      _stream(stream)))


def prefill_chunk(shape, sel, max_chunk, q_chunk, chunk_lens, k_pool, v_pool, block_table, seq_lens,
                  sel_idx, sel_count, out, ws, stream=None):
    lib = load_library()
    _check(lib.tokenselect_prefill_chunk(ctypes.byref(shape), ctypes.byref(sel), int(max_chunk),
                                         _ptr(q_chunk), _ptr(chunk_lens), _ptr(k_pool), _ptr(v_pool),
                                         _ptr(block_table), _ptr(seq_lens), _ptr(sel_idx),
                                         _ptr(sel_count), _ptr(out), _ptr(ws), ws.numel(),
                                         _stream(stream)))


# ---------------------------------------------------------------- selection-function ablations
SELECT_SOFT_VOTE, SELECT_NAIVE_TOPK, SELECT_HARD_VOTE, SELECT_BLOCK = range(4)


def ablation_workspace_size(shape: Shape, sel: Select, fn: int, block: int = 1) -> int:
    return int(load_library().tokenselect_ablation_workspace_size(ctypes.byref(shape), ctypes.byref(sel),
                                                                  int(fn), int(block)))


def alloc_ablation_workspace(shape: Shape, sel: Select, fn: int, block: int = 1, device="cuda") -> torch.Tensor:
    n = ablation_workspace_size(shape, sel, fn, block)
    if n == 0:
        raise TokenSelectError(TS_ERR_INVALID_ARG, load_library().tokenselect_last_error().decode())
    return torch.empty(n, dtype=torch.uint8, device=device)


def select_ablation(shape, sel, fn, block, logits, head_stats, seq_lens, score, sel_idx, sel_count, ws,
                    stream=None):
    lib = load_library()
    _check(lib.tokenselect_select_ablation(ctypes.byref(shape), ctypes.byref(sel), int(fn), int(block),
                                           _ptr(logits), _ptr(head_stats), _ptr(seq_lens), _ptr(score),
                                           _ptr(sel_idx), _ptr(sel_count), _ptr(ws), ws.numel(),
                                           _stream(stream)))


# ---------------------------------------------------------------- input checks
def validate(shape, block_table, seq_lens, num_pool_pages: int, report=None, stream=None) -> torch.Tensor:
    """tokenselect_validate: returns the device report (int64 [4]: violations, first
    (request << 32 | page) key, length violations, sum of lengths); read it after
    synchronising. `report` may be given to reuse a buffer."""
    lib = load_library()
    if report is None:
        report = torch.empty(4, dtype=torch.int64, device=seq_lens.device)
    _check(lib.tokenselect_validate(ctypes.byref(shape), _ptr(block_table), _ptr(seq_lens),
                                    int(num_pool_pages), _ptr(report), _stream(stream)))
    return report


def validate_selection(shape, sel, seq_lens, sel_idx, sel_count, report=None, stream=None) -> torch.Tensor:
    """tokenselect_validate_selection: returns the device report (int64 [4]: violations,
    first (request << 32 | entry) key, count violations, sum of the in-range counts);
    read it after synchronising."""
    lib = load_library()
    if report is None:
        report = torch.empty(4, dtype=torch.int64, device=seq_lens.device)
    _check(lib.tokenselect_validate_selection(ctypes.byref(shape), ctypes.byref(sel), _ptr(seq_lens),
                                              _ptr(sel_idx), _ptr(sel_count), _ptr(report), _stream(stream)))
    return report
