"""Python binding of libqsa (QSA attention over an int8 KV cache, MI355X / gfx950).

Argument marshalling only: every function checks dtypes, devices, contiguity and sizes of torch tensors (the sizes
against the dims, row counts, k, n_blocks and max_chunks the C side will index them by), passes their device
pointers and the current HIP stream to the C ABI declared in include/qsa.h, and raises QSAError on a non-zero
status. No torch operator runs on the compute path; PyTorch supplies device memory and streams.

The library is the in-tree ``libqsa.so``; importing this package raises if it has not been built (there is no
fallback implementation).
"""
from __future__ import annotations

import ctypes
import dataclasses
import os
from typing import Optional, Sequence

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libqsa.so")

QSA_OK = 0
STATUS_NAMES = {0: "QSA_OK", -1: "QSA_ERR_NULL", -2: "QSA_ERR_SHAPE", -3: "QSA_ERR_UNSUPPORTED",
                -4: "QSA_ERR_SCRATCH", -5: "QSA_ERR_RANGE", -6: "QSA_ERR_LAUNCH"}
BLOCK = 64
NOALLOC_SCRATCH_BYTES = 8 << 20   # QSA_NOALLOC_SCRATCH_BYTES in include/qsa.h


class QSAError(RuntimeError):
    def __init__(self, fn, status):
        self.status = status
        super().__init__(f"{fn} failed: {STATUS_NAMES.get(status, status)} ({_lib().qsa_status_str(status).decode()})")


class _Dims(ctypes.Structure):
    _fields_ = [("n_q_heads", ctypes.c_int32), ("n_kv_heads", ctypes.c_int32), ("head_dim", ctypes.c_int32),
                ("block_cells", ctypes.c_int32)]


class _Pool(ctypes.Structure):
    _fields_ = [("k", ctypes.c_void_p), ("k_scale", ctypes.c_void_p), ("v", ctypes.c_void_p),
                ("v_scale", ctypes.c_void_p), ("index", ctypes.c_void_p), ("capacity", ctypes.c_int32),
                ("n_valid", ctypes.c_int32), ("v_bits", ctypes.c_int32)]


class _Partials(ctypes.Structure):
    _fields_ = [("m", ctypes.c_void_p), ("l", ctypes.c_void_p), ("o", ctypes.c_void_p), ("empty", ctypes.c_void_p),
                ("max_chunks", ctypes.c_int32)]


_L = None


def _lib():
    global _L
    if _L is None:
        if not os.path.exists(LIB_PATH):
            raise ImportError(f"libqsa.so is not built ({LIB_PATH}); run __graft_entry__.build() or "
                              f"python -m sparse_top_attention_amd.build")
        L = ctypes.CDLL(LIB_PATH)
        P, I32, SZ = ctypes.c_void_p, ctypes.c_int32, ctypes.c_size_t
        PP, PD, PPart = ctypes.POINTER(_Pool), _Dims, ctypes.POINTER(_Partials)
        L.qsa_block_index.argtypes = [PP, PD, I32, I32, P, P]
        L.qsa_block_scores.argtypes = [P, P, I32, PP, PD, I32, P, P]
        L.qsa_topk_scratch_bytes.argtypes = [I32, I32, I32]
        L.qsa_topk_scratch_bytes.restype = SZ
        L.qsa_topk.argtypes = [P, I32, I32, I32, P, P, P, SZ, P]
        L.qsa_attn_chunk.argtypes = [P, P, I32, PP, I32, P, PD, P, P, I32, I32, I32, ctypes.c_float, PPart, P]
        L.qsa_attn_merge.argtypes = [PPart, I32, PD, I32, P, P, P, P]
        L.qsa_prompt_scratch_bytes.argtypes = [I32, I32, PD]
        L.qsa_prompt_scratch_bytes.restype = SZ
        L.qsa_prompt_attn.argtypes = [P, I32, I32, PP, PD, ctypes.c_float, P, P, SZ, P]
        L.qsa_kv_append.argtypes = [PP, I32, P, PD, P, P, P, I32, P]
        L.qsa_decode_select.argtypes = [P, P, I32, PP, I32, P, PD, I32, I32, P, P, P, P]
        L.qsa_decode_layer_scratch_bytes.argtypes = [I32, PD, I32, I32, I32]
        L.qsa_decode_layer_scratch_bytes.restype = SZ
        L.qsa_decode_layer.argtypes = [P, P, I32, PP, I32, P, PD, I32, I32, I32, ctypes.c_float, P, P, P, P, P, P,
                                       SZ, P]
        L.qsa_decode_layer_noalloc.argtypes = [P, P, I32, PP, I32, P, PD, I32, I32, I32, ctypes.c_float, P, P, P, P,
                                               P, P]
        L.qsa_status_str.argtypes = [I32]
        L.qsa_status_str.restype = ctypes.c_char_p
        for fn in ("qsa_block_index", "qsa_block_scores", "qsa_topk", "qsa_attn_chunk", "qsa_attn_merge",
                   "qsa_prompt_attn", "qsa_decode_layer", "qsa_decode_select", "qsa_kv_append",
                   "qsa_decode_layer_noalloc"):
            getattr(L, fn).restype = I32
        _L = L
    return _L


def lib_handle():
    """The loaded ctypes library (loads it on first use)."""
    return _lib()


# ----------------------------------------------------------------------------------------------- helpers
def _ptr(t: Optional[torch.Tensor], dtype, name, allow_none=False):
    if t is None:
        if allow_none:
            return None
        raise ValueError(f"{name} is required")
    if t.dtype != dtype:
        raise TypeError(f"{name}: expected {dtype}, got {t.dtype}")
    if not t.is_cuda:
        raise ValueError(f"{name}: expected a GPU tensor")
    if not t.is_contiguous():
        raise ValueError(f"{name}: expected a contiguous tensor")
    return t.data_ptr()


def _need(t: Optional[torch.Tensor], n: int, name: str):
    """The C side indexes t as n elements (its size cannot be checked on the device): refuse a smaller tensor."""
    if t is not None and t.numel() < n:
        raise ValueError(f"{name}: the call reads or writes {n} elements, the tensor holds {t.numel()}")


def _shape(t: Optional[torch.Tensor], shape, name: str):
    if t is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name}: expected shape {tuple(shape)}, got {tuple(t.shape)}")


def _rows_of(q: torch.Tensor, dims: "Dims", name="q"):
    """q is [n_rows][n_q_heads][head_dim] (or [n_rows][n_q_heads * head_dim])."""
    if q.dim() < 1:
        raise ValueError(f"{name}: expected [n_rows][n_q_heads][head_dim]")
    n = q.shape[0]
    _need(q, n * dims.n_q_heads * dims.head_dim, name)
    if q.numel() != n * dims.n_q_heads * dims.head_dim:
        raise ValueError(f"{name}: expected {n} x {dims.n_q_heads} x {dims.head_dim} elements, got {q.numel()}")
    return n


def _check_pools(pools: Sequence["Pool"], dims: "Dims", need_index=False):
    if len(pools) == 0:
        raise ValueError("at least one pool is required")
    for p in pools:
        p.check(dims, need_index)


def _pool_array(pools: Sequence["Pool"]):
    return (_Pool * len(pools))(*[p.c() for p in pools])


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return ctypes.c_void_p(stream.cuda_stream)


def _check(fn, status):
    if status != QSA_OK:
        raise QSAError(fn, status)


@dataclasses.dataclass
class Dims:
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    block_cells: int = BLOCK

    def c(self):
        return _Dims(self.n_q_heads, self.n_kv_heads, self.head_dim, self.block_cells)


@dataclasses.dataclass
class Pool:
    """Device tensors of one int8 KV pool: k int8 [n_kv][cap][d]; v int8 [n_kv][cap][d] (v_bits 8) or
    [n_kv][cap][d/2] bytes of two 4-bit codes (v_bits 4, K8V4); k_scale, v_scale f32 [n_kv][cap][d/64];
    index f32 [n_kv][ceil(cap/64)][d] (optional, needed by the selection calls)."""
    k: torch.Tensor
    k_scale: torch.Tensor
    v: torch.Tensor
    v_scale: torch.Tensor
    n_valid: int
    index: Optional[torch.Tensor] = None
    v_bits: int = 8

    @property
    def capacity(self):
        return self.k.shape[1]

    def check(self, dims: "Dims", need_index=False):
        """Every tensor's shape against dims and the capacity k implies (the kernels index them by those)."""
        if self.k.dim() != 3:
            raise ValueError("k: expected [n_kv_heads][capacity][head_dim]")
        n_kv, cap, d = dims.n_kv_heads, self.capacity, dims.head_dim
        _shape(self.k, (n_kv, cap, d), "k")
        _shape(self.k_scale, (n_kv, cap, max(d // 64, 1)), "k_scale")
        _shape(self.v, (n_kv, cap, d if self.v_bits in (0, 8) else d // 2), "v")
        _shape(self.v_scale, (n_kv, cap, max(d // 64, 1)), "v_scale")
        _shape(self.index, (n_kv, -(-cap // BLOCK), d), "index")
        if need_index and self.index is None:
            raise ValueError("index: the selection calls need the pool's block index")
        if not 0 <= self.n_valid <= cap:
            raise ValueError(f"n_valid {self.n_valid} outside [0, capacity {cap}]")

    def c(self):
        return _Pool(_ptr(self.k, torch.int8, "k"), _ptr(self.k_scale, torch.float32, "k_scale"),
                     _ptr(self.v, torch.int8, "v"), _ptr(self.v_scale, torch.float32, "v_scale"),
                     _ptr(self.index, torch.float32, "index", allow_none=True), self.capacity, self.n_valid,
                     self.v_bits)


@dataclasses.dataclass
class Partials:
    """Chunk partials: m, l f32 [n_rows][Hq][max_chunks]; o f32 [n_rows][Hq][max_chunks][d]; empty u8."""
    m: torch.Tensor
    l: torch.Tensor
    o: torch.Tensor
    empty: torch.Tensor

    @property
    def max_chunks(self):
        return self.m.shape[-1]

    @staticmethod
    def empty_like_shape(n_rows, n_q_heads, max_chunks, head_dim, device="cuda"):
        return Partials(torch.empty(n_rows, n_q_heads, max_chunks, dtype=torch.float32, device=device),
                        torch.empty(n_rows, n_q_heads, max_chunks, dtype=torch.float32, device=device),
                        torch.empty(n_rows, n_q_heads, max_chunks, head_dim, dtype=torch.float32, device=device),
                        torch.empty(n_rows, n_q_heads, max_chunks, dtype=torch.uint8, device=device))

    def check(self, n_rows: int, dims: "Dims"):
        """m, l, empty [>= n_rows][n_q_heads][max_chunks] and o [...][head_dim], the strides the kernels use."""
        mc = self.max_chunks
        _need(self.m, n_rows * dims.n_q_heads * mc, "partials m")
        _need(self.l, n_rows * dims.n_q_heads * mc, "partials l")
        _need(self.empty, n_rows * dims.n_q_heads * mc, "partials empty")
        _need(self.o, n_rows * dims.n_q_heads * mc * dims.head_dim, "partials o")

    def c(self):
        return _Partials(_ptr(self.m, torch.float32, "m"), _ptr(self.l, torch.float32, "l"),
                         _ptr(self.o, torch.float32, "o"), _ptr(self.empty, torch.uint8, "empty"), self.max_chunks)


# --------------------------------------------------------------------------------------------- the calls
def qsa_block_index(pool: Pool, dims: Dims, cell_begin: int, cell_end: int, index: torch.Tensor, stream=None):
    pool.check(dims)
    _shape(index, (dims.n_kv_heads, -(-pool.capacity // BLOCK), dims.head_dim), "index")
    p = pool.c()
    _check("qsa_block_index", _lib().qsa_block_index(ctypes.byref(p), dims.c(), cell_begin, cell_end,
                                                     _ptr(index, torch.float32, "index"), _stream(stream)))
    return index


def qsa_block_scores(q, pos, pool: Pool, dims: Dims, n_blocks: int, scores, stream=None):
    pool.check(dims, need_index=True)
    n = _rows_of(q, dims)
    _need(pos, n, "pos")
    _need(scores, n * dims.n_kv_heads * n_blocks, "scores")
    p = pool.c()
    _check("qsa_block_scores", _lib().qsa_block_scores(_ptr(q, torch.float32, "q"), _ptr(pos, torch.int32, "pos"),
                                                       n, ctypes.byref(p), dims.c(), n_blocks,
                                                       _ptr(scores, torch.float32, "scores"), _stream(stream)))
    return scores


def qsa_topk_scratch_bytes(n_rows, width, k):
    return _lib().qsa_topk_scratch_bytes(n_rows, width, k)


def qsa_topk(scores, k, ids, counts, scratch=None, stream=None):
    width = scores.shape[-1]
    n_rows = scores.numel() // width if width else 0
    _need(ids, n_rows * k, "ids")
    _need(counts, n_rows, "counts")
    sp = None if scratch is None else _ptr(scratch, torch.uint8, "scratch")
    nbytes = 0 if scratch is None else scratch.numel()
    _check("qsa_topk", _lib().qsa_topk(_ptr(scores, torch.float32, "scores"), n_rows, width, k,
                                       _ptr(ids, torch.int32, "ids"), _ptr(counts, torch.int32, "counts"),
                                       sp, nbytes, _stream(stream)))
    return ids, counts


def qsa_attn_chunk(q, pos, pools: Sequence[Pool], dims: Dims, out: Partials, n_chunks: int, sm_scale: float = 1.0,
                   row_pool=None, ids=None, counts=None, blocks_per_chunk: int = 1, stream=None):
    _check_pools(pools, dims)
    n = _rows_of(q, dims)
    k = ids.shape[-1] if ids is not None else 0
    _need(pos, n, "pos")
    _need(row_pool, n, "row_pool")
    _need(ids, n * dims.n_kv_heads * k, "ids")
    _need(counts, n * dims.n_kv_heads, "counts")
    out.check(n, dims)
    part = out.c()
    arr = _pool_array(pools)
    _check("qsa_attn_chunk", _lib().qsa_attn_chunk(
        _ptr(q, torch.float32, "q"), _ptr(pos, torch.int32, "pos"), n, arr, len(pools),
        _ptr(row_pool, torch.int32, "row_pool", allow_none=True), dims.c(),
        _ptr(ids, torch.int32, "ids", allow_none=True), _ptr(counts, torch.int32, "counts", allow_none=True), k,
        blocks_per_chunk, n_chunks, sm_scale, ctypes.byref(part), _stream(stream)))
    return out


def qsa_attn_merge(part: Partials, dims: Dims, n_chunks: int, out, lse=None, n_active=None, stream=None):
    n = part.m.shape[0]
    part.check(n, dims)
    _need(out, n * dims.n_q_heads * dims.head_dim, "out")
    _need(lse, n * dims.n_q_heads, "lse")
    _need(n_active, n, "n_active")
    pc = part.c()
    _check("qsa_attn_merge", _lib().qsa_attn_merge(
        ctypes.byref(pc), n, dims.c(), n_chunks, _ptr(n_active, torch.int32, "n_active", True),
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse", allow_none=True), _stream(stream)))
    return out


def qsa_kv_append(pools: Sequence[Pool], dims: Dims, k_new, v_new, cells, row_pool=None, stream=None):
    _check_pools(pools, dims)
    n = k_new.shape[0]
    _need(k_new, n * dims.n_kv_heads * dims.head_dim, "k_new")
    _need(v_new, n * dims.n_kv_heads * dims.head_dim, "v_new")
    _need(cells, n, "cells")
    _need(row_pool, n, "row_pool")
    arr = _pool_array(pools)
    _check("qsa_kv_append", _lib().qsa_kv_append(
        arr, len(pools), _ptr(row_pool, torch.int32, "row_pool", allow_none=True), dims.c(),
        _ptr(k_new, torch.float32, "k_new"), _ptr(v_new, torch.float32, "v_new"), _ptr(cells, torch.int32, "cells"),
        k_new.shape[0], _stream(stream)))


def qsa_decode_select(q, pos, pools: Sequence[Pool], dims: Dims, n_blocks: int, k: int, ids, counts, scores=None,
                      row_pool=None, stream=None):
    _check_pools(pools, dims, need_index=True)
    n = _rows_of(q, dims)
    _need(pos, n, "pos")
    _need(row_pool, n, "row_pool")
    _need(ids, n * dims.n_kv_heads * k, "ids")
    _need(counts, n * dims.n_kv_heads, "counts")
    _need(scores, n * dims.n_kv_heads * n_blocks, "scores")
    arr = _pool_array(pools)
    _check("qsa_decode_select", _lib().qsa_decode_select(
        _ptr(q, torch.float32, "q"), _ptr(pos, torch.int32, "pos"), n, arr, len(pools),
        _ptr(row_pool, torch.int32, "row_pool", allow_none=True), dims.c(), n_blocks, k,
        _ptr(scores, torch.float32, "scores", allow_none=True), _ptr(ids, torch.int32, "ids"),
        _ptr(counts, torch.int32, "counts"), _stream(stream)))
    return ids, counts


def qsa_decode_layer_scratch_bytes(n_rows, dims: Dims, n_blocks, k, n_chunks):
    return _lib().qsa_decode_layer_scratch_bytes(n_rows, dims.c(), n_blocks, k, n_chunks)


def qsa_decode_layer(q, pos, pools: Sequence[Pool], dims: Dims, n_blocks: int, k: int, n_chunks: int, out, lse=None,
                     sm_scale: float = 1.0, row_pool=None, scores=None, ids=None, counts=None, scratch=None,
                     stream=None):
    _check_pools(pools, dims, need_index=True)
    n = _rows_of(q, dims)
    _need(pos, n, "pos")
    _need(row_pool, n, "row_pool")
    _need(out, n * dims.n_q_heads * dims.head_dim, "out")
    _need(lse, n * dims.n_q_heads, "lse")
    _need(scores, n * dims.n_kv_heads * n_blocks, "scores")
    _need(ids, n * dims.n_kv_heads * k, "ids")
    _need(counts, n * dims.n_kv_heads, "counts")
    sp = None if scratch is None else _ptr(scratch, torch.uint8, "scratch")
    nbytes = 0 if scratch is None else scratch.numel()
    arr = _pool_array(pools)
    _check("qsa_decode_layer", _lib().qsa_decode_layer(
        _ptr(q, torch.float32, "q"), _ptr(pos, torch.int32, "pos"), n, arr, len(pools),
        _ptr(row_pool, torch.int32, "row_pool", allow_none=True), dims.c(), n_blocks, k, n_chunks, sm_scale,
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse", allow_none=True),
        _ptr(scores, torch.float32, "scores", allow_none=True), _ptr(ids, torch.int32, "ids", allow_none=True),
        _ptr(counts, torch.int32, "counts", allow_none=True), sp, nbytes, _stream(stream)))
    return out


def qsa_decode_layer_noalloc(q, pos, pools: Sequence[Pool], dims: Dims, n_blocks: int, k: int, n_chunks: int, out,
                             lse=None, sm_scale: float = 1.0, row_pool=None, scores=None, ids=None, counts=None,
                             stream=None):
    """qsa_decode_layer with the library's per-device static scratch (no scratch argument, nothing allocated)."""
    _check_pools(pools, dims, need_index=True)
    n = _rows_of(q, dims)
    _need(pos, n, "pos")
    _need(row_pool, n, "row_pool")
    _need(out, n * dims.n_q_heads * dims.head_dim, "out")
    _need(lse, n * dims.n_q_heads, "lse")
    _need(scores, n * dims.n_kv_heads * n_blocks, "scores")
    _need(ids, n * dims.n_kv_heads * k, "ids")
    _need(counts, n * dims.n_kv_heads, "counts")
    arr = _pool_array(pools)
    _check("qsa_decode_layer_noalloc", _lib().qsa_decode_layer_noalloc(
        _ptr(q, torch.float32, "q"), _ptr(pos, torch.int32, "pos"), n, arr, len(pools),
        _ptr(row_pool, torch.int32, "row_pool", allow_none=True), dims.c(), n_blocks, k, n_chunks, sm_scale,
        _ptr(out, torch.float32, "out"), _ptr(lse, torch.float32, "lse", allow_none=True),
        _ptr(scores, torch.float32, "scores", allow_none=True), _ptr(ids, torch.int32, "ids", allow_none=True),
        _ptr(counts, torch.int32, "counts", allow_none=True), _stream(stream)))
    return out


def qsa_prompt_scratch_bytes(n_q, pos0, dims: Dims):
    return _lib().qsa_prompt_scratch_bytes(n_q, pos0, dims.c())


def qsa_prompt_attn(q, pos0: int, pool: Pool, dims: Dims, out, sm_scale: float = 1.0, scratch=None, stream=None):
    pool.check(dims)
    n = _rows_of(q, dims)
    _need(out, n * dims.n_q_heads * dims.head_dim, "out")
    p = pool.c()
    sp = None if scratch is None else _ptr(scratch, torch.uint8, "scratch")
    nbytes = 0 if scratch is None else scratch.numel()
    _check("qsa_prompt_attn", _lib().qsa_prompt_attn(_ptr(q, torch.float32, "q"), n, pos0,
                                                     ctypes.byref(p), dims.c(), sm_scale,
                                                     _ptr(out, torch.float32, "out"), sp, nbytes, _stream(stream)))
    return out


def qsa_status_str(status: int) -> str:
    return _lib().qsa_status_str(status).decode()


__all__ = ["Dims", "Pool", "Partials", "QSAError", "qsa_block_index", "qsa_block_scores", "qsa_topk_scratch_bytes",
           "qsa_topk", "qsa_attn_chunk", "qsa_attn_merge", "qsa_prompt_scratch_bytes", "qsa_prompt_attn",
           "qsa_decode_select", "qsa_decode_layer_scratch_bytes", "qsa_decode_layer", "qsa_decode_layer_noalloc",
           "qsa_kv_append",
           "qsa_status_str", "lib_handle"]
