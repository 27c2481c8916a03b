"""FP64 CPU reference for QSA attention -- TEST INFRASTRUCTURE ONLY.

Thin numpy/ctypes wrappers over ``qsa_oracle.c`` (single-threaded, FP64). Only the test suite, the smoke check and
the benchmark's CPU-baseline leg may import this package. It shares no code with the GPU library.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "qsa_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
BLOCK = 64

GCC_CMD = ["gcc", "-O2", "-std=c11", "-Wall", "-Wextra", "-fPIC", "-shared", _SRC, "-o", _LIB, "-lm"]


def build():
    """Compile the oracle (plain C, -O2, no fast-math, no threads)."""
    subprocess.run(GCC_CMD, check=True)


_lib = None


def lib():
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = ctypes.CDLL(_LIB)
        _declare(_lib)
    return _lib


P = ctypes.c_void_p
I32 = ctypes.c_int32
I64 = ctypes.c_int64
F64 = ctypes.c_double


def _declare(L):
    L.orc_block_index.argtypes = [P, P, I32, I32, I32, I32, I32, I32, P]
    L.orc_block_scores.argtypes = [P, P, I32, I32, I32, I32, P, I32, I32, I32, I32, P]
    L.orc_topk.argtypes = [P, I32, I32, I32, P, P]
    L.orc_attn_one.argtypes = [P, P, I32, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, I32, F64, P, P, I32]
    L.orc_attn.argtypes = [P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, I32, F64, P, P, I32]
    L.orc_chunk_partials.argtypes = [P, P, I32, P, P, P, P, I32, I32, I32, I32, I32, I32, P, P, I32, I32, I32, F64,
                                     P, P, P, P, I32]
    L.orc_merge.argtypes = [P, P, P, P, I32, I32, I32, I32, P, P, P]
    L.orc_split24.argtypes = [P, I64, P, P, P]
    L.orc_split24.restype = ctypes.c_int
    L.orc_quant24.argtypes = [P, I64, F64, P]
    L.orc_encode_group.argtypes = [P, I32, P, P]
    L.orc_kv_append.argtypes = [P, P, P, P, I32, I32, I32, I32, P, P, P, I32, I32]
    L.orc_encode_group4.argtypes = [P, I32, P, P]


def _c(a, dtype):
    a = np.ascontiguousarray(a, dtype=dtype)
    return a


def _p(a):
    return None if a is None else a.ctypes.data_as(ctypes.c_void_p)


def _v_bits(pool):
    return int(getattr(pool, "v_bits", 8))


def _pool_args(pool):
    k = _c(pool.k, np.int8)
    ks = _c(pool.ks, np.float32)
    v = _c(pool.v, np.int8)
    vs = _c(pool.vs, np.float32)
    return (k, ks, v, vs)


def block_index(pool, n_blocks=None):
    """r [n_kv][n_blocks][d] float64, the mean dequantised key of each block's valid cells."""
    n_kv, cap, d = pool.k.shape
    if n_blocks is None:
        n_blocks = -(-pool.n_valid // BLOCK)
    k, ks = _c(pool.k, np.int8), _c(pool.ks, np.float32)
    r = np.zeros((n_kv, n_blocks, d), np.float64)
    lib().orc_block_index(_p(k), _p(ks), n_kv, cap, pool.n_valid, d, BLOCK, n_blocks, _p(r))
    return r


def block_scores(q, pos, r, n_kv, n_valid, n_blocks):
    """s [n_rows][n_kv][n_blocks] float64 from q [n_rows][Hq][d] and an index r [n_kv][r_blocks][d]."""
    q = _c(q, np.float32)
    pos = _c(pos, np.int32)
    r = _c(r, np.float64)
    n_rows, n_qh, d = q.shape
    s = np.zeros((n_rows, n_kv, n_blocks), np.float64)
    lib().orc_block_scores(_p(q), _p(pos), n_rows, n_qh, n_kv, d, _p(r), r.shape[1], n_valid, BLOCK, n_blocks,
                           _p(s))
    return s


def topk(s, k):
    """ids [R][k] int32 (ascending, -1 padded) and counts [R] for score rows s [R][W] (any float dtype)."""
    s = _c(s, np.float64)
    R, W = s.reshape(-1, s.shape[-1]).shape
    ids = np.zeros((R, k), np.int32)
    counts = np.zeros(R, np.int32)
    lib().orc_topk(_p(s), R, W, k, _p(ids), _p(counts))
    return ids, counts


def attn(q, pos, pool, n_kv, ids=None, counts=None, topk_=0, sm_scale=1.0):
    """out [n_rows][Hq][d], lse [n_rows][Hq] in float64; ids [n_rows][n_kv][k] or None for dense attention."""
    q = _c(q, np.float32)
    pos = _c(pos, np.int32)
    n_rows, n_qh, d = q.shape
    k, ks, v, vs = _pool_args(pool)
    if ids is not None:
        ids = _c(ids, np.int32)
        counts = _c(counts, np.int32)
        topk_ = ids.shape[-1]
    out = np.zeros((n_rows, n_qh, d), np.float64)
    lse = np.zeros((n_rows, n_qh), np.float64)
    lib().orc_attn(_p(q), _p(pos), n_rows, _p(k), _p(ks), _p(v), _p(vs), pool.capacity, pool.n_valid, n_qh, n_kv,
                   d, BLOCK, _p(ids), _p(counts), topk_, sm_scale, _p(out), _p(lse), _v_bits(pool))
    return out, lse


def attn_one(q, pos, i, h, pool, n_kv, ids=None, counts=None, sm_scale=1.0):
    """One (row, q head) of ``attn``: (out [d], lse)."""
    q = _c(q, np.float32)
    pos = _c(pos, np.int32)
    n_rows, n_qh, d = q.shape
    k, ks, v, vs = _pool_args(pool)
    topk_ = 0
    if ids is not None:
        ids = _c(ids, np.int32)
        counts = _c(counts, np.int32)
        topk_ = ids.shape[-1]
    out = np.zeros(d, np.float64)
    lse = np.zeros(1, np.float64)
    lib().orc_attn_one(_p(q), _p(pos), i, h, _p(k), _p(ks), _p(v), _p(vs), pool.capacity, pool.n_valid, n_qh,
                       n_kv, d, BLOCK, _p(ids), _p(counts), topk_, sm_scale, _p(out), _p(lse), _v_bits(pool))
    return out, float(lse[0])


def chunk_partials(q, pos, pool, n_kv, n_chunks, ids=None, counts=None, bpc=1, sm_scale=1.0):
    """(m, l, o, empty) with m, l [n_rows][Hq][S], o [n_rows][Hq][S][d] (float64), empty uint8."""
    q = _c(q, np.float32)
    pos = _c(pos, np.int32)
    n_rows, n_qh, d = q.shape
    k, ks, v, vs = _pool_args(pool)
    topk_ = 0
    if ids is not None:
        ids = _c(ids, np.int32)
        counts = _c(counts, np.int32)
        topk_ = ids.shape[-1]
    m = np.zeros((n_rows, n_qh, n_chunks), np.float64)
    l = np.zeros_like(m)
    o = np.zeros((n_rows, n_qh, n_chunks, d), np.float64)
    e = np.zeros((n_rows, n_qh, n_chunks), np.uint8)
    lib().orc_chunk_partials(_p(q), _p(pos), n_rows, _p(k), _p(ks), _p(v), _p(vs), pool.capacity, pool.n_valid,
                             n_qh, n_kv, d, BLOCK, _p(ids), _p(counts), topk_, bpc, n_chunks, sm_scale, _p(m), _p(l),
                             _p(o), _p(e), _v_bits(pool))
    return m, l, o, e


def merge(m, l, o, empty, n_active=None):
    """(out [n_rows][Hq][d], lse [n_rows][Hq]) from chunk partials."""
    m = _c(m, np.float64)
    l = _c(l, np.float64)
    o = _c(o, np.float64)
    empty = _c(empty, np.uint8)
    n_rows, n_qh, S, d = o.shape
    if n_active is not None:
        n_active = _c(n_active, np.int32)
    out = np.zeros((n_rows, n_qh, d), np.float64)
    lse = np.zeros((n_rows, n_qh), np.float64)
    lib().orc_merge(_p(m), _p(l), _p(o), _p(empty), n_rows, n_qh, S, d, _p(n_active), _p(out), _p(lse))
    return out, lse


def split24(X):
    """Balanced three-digit split of integers X: (h, l, m) with X = 65536 h + 256 l + m."""
    X = _c(X, np.int32)
    n = X.size
    h = np.zeros(n, np.int32)
    l = np.zeros(n, np.int32)
    m = np.zeros(n, np.int32)
    rc = lib().orc_split24(_p(X), n, _p(h), _p(l), _p(m))
    if rc != 0:
        raise ValueError("value outside the three-digit range")
    return h.reshape(X.shape), l.reshape(X.shape), m.reshape(X.shape)


def quant24(x, amax):
    x = _c(x, np.float64)
    X = np.zeros(x.size, np.int32)
    lib().orc_quant24(_p(x), x.size, float(amax), _p(X))
    return X.reshape(x.shape)


def full_selection(pos, n_kv, n_valid, n_blocks_k):
    """Dense selection (every eligible block) as ids/counts, used where k >= the number of blocks."""
    n_rows = len(pos)
    nb = -(-n_valid // BLOCK)
    ids = -np.ones((n_rows, n_kv, n_blocks_k), np.int32)
    counts = np.zeros((n_rows, n_kv), np.int32)
    for i in range(n_rows):
        elig = [b for b in range(nb) if b * BLOCK <= pos[i]][:n_blocks_k]
        for g in range(n_kv):
            ids[i, g, :len(elig)] = elig
            counts[i, g] = len(elig)
    return ids, counts


def encode_group(x):
    """int8 codes and the fp32 scale of one group of values (fp32 decisions, see orc_encode_group)."""
    x = _c(x, np.float32)
    codes = np.zeros(x.shape[0], np.int8)
    scale = np.zeros(1, np.float32)
    lib().orc_encode_group(_p(x), x.shape[0], _p(codes), _p(scale))
    return codes, float(scale[0])


def encode_group4(x):
    """4-bit codes (as int8 in [-7, 7]) and the fp32 scale of one group (see orc_encode_group4)."""
    x = _c(x, np.float32)
    codes = np.zeros(x.shape[0], np.int8)
    scale = np.zeros(1, np.float32)
    lib().orc_encode_group4(_p(x), x.shape[0], _p(codes), _p(scale))
    return codes, float(scale[0])


def kv_append(pool, k_new, v_new, cells, n_valid=None):
    """A copy of ``pool`` (a synth.Pool) with rows k_new, v_new [n_rows][n_kv][d] appended at cells [n_rows];
    n_valid is the count after the append (default: the pool's)."""
    import copy
    out = copy.copy(pool)
    out.k, out.ks, out.v, out.vs = (np.array(a, copy=True, order="C") for a in (pool.k, pool.ks, pool.v, pool.vs))
    out.n_valid = pool.n_valid if n_valid is None else n_valid
    n_kv, cap, d = out.k.shape
    kn, vn = _c(k_new, np.float32), _c(v_new, np.float32)   # d from K: a K8V4 pool's V rows are d/2 bytes
    cl = _c(cells, np.int32)
    lib().orc_kv_append(_p(out.k), _p(out.ks), _p(out.v), _p(out.vs), n_kv, cap, out.n_valid, d, _p(kn), _p(vn),
                        _p(cl), cl.shape[0], _v_bits(pool))
    return out
