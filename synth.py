"""Seeded synthetic inputs for the QSA decode and prompt-chunk workloads.

This module only draws random numbers and lays them out; it holds none of the attention arithmetic. Both the
GPU library's tests/bench and the FP64 reference read their inputs from here, so the two sides always see the
same bytes.

Shapes follow the workloads the pages measure:
  * int8 K/V codes with one fp32 scale per (KV head, cell, 64-dim group) -- #1367 (prompt attention on INT8
    tensor cores), "What it does", and the Volta prompt-kernel PR, where a 64-dim group is one int8 scale group;
  * 24 q heads over 4 KV heads and a 200,000-cell capacity -- #2806 (sycl decode QSA selection), kernel table;
  * a 4-row verify window, a 2-slot batch window, the drafter's 32K window of 512 chunks, and a 2,048-query prompt
    chunk at the end of a 32K context -- #2075 (bench table), #2806 (kernel table), #1367 (accuracy table).

Value distributions (the pages give none): codes uniform on [-127, 127], scales uniform on [0.005, 0.02),
q ~ N(0, 1)/sqrt(head_dim) drawn in float64 and rounded to float32. Cells past ``n_valid`` hold poison (codes
-128, NaN scales) for parity runs, so any read outside the valid range shows up, or zeros for timing runs.

Pool layout: codes ``[n_kv][capacity][d]`` int8, scales ``[n_kv][capacity][d // 64]`` float32. A K8V4 pool
(``v_bits=4``, a cache format the pages list beside int8 without its layout) keeps int8 K and stores V as signed
4-bit codes (uniform on [-7, 7]) packed two per byte, ``[n_kv][capacity][d // 2]``, dim 2j in the low nibble.
"""
from __future__ import annotations

import dataclasses
import math

import numpy as np

GROUP = 64          # dims per int8 scale group
BLOCK = 64          # cells per selection block
POISON_CODE = -128


@dataclasses.dataclass
class Pool:
    k: np.ndarray        # int8  [n_kv][cap][d]
    ks: np.ndarray       # f32   [n_kv][cap][d/64]
    v: np.ndarray        # int8  [n_kv][cap][d] (v_bits 8) or bytes [n_kv][cap][d/2] of two 4-bit codes (v_bits 4)
    vs: np.ndarray       # f32   [n_kv][cap][d/64]
    capacity: int
    n_valid: int
    v_bits: int = 8


@dataclasses.dataclass
class Workload:
    name: str
    n_q_heads: int
    n_kv_heads: int
    head_dim: int
    pools: list          # list[Pool]
    q: np.ndarray        # f32 [n_rows][Hq][d]
    pos: np.ndarray      # int32 [n_rows]
    row_pool: np.ndarray  # int32 [n_rows]
    topk: int            # 0 = dense (no selection)
    n_chunks: int        # chunk count the pages' workload uses (parity default)
    blocks_per_chunk: int  # dense mode only
    n_active: int        # dense mode: chunks holding cells
    sm_scale: float
    prompt: bool = False
    pos0: int = 0


def _codes(rng, shape):
    return rng.integers(-127, 128, size=shape, dtype=np.int8)


def _scales(rng, shape):
    return rng.uniform(0.005, 0.02, size=shape).astype(np.float32)


def pack_v4(codes):
    """Signed 4-bit codes [..., d] (in [-8, 7]) -> bytes [..., d/2] as int8: dim 2j in the low nibble, 2j + 1 in the
    high nibble (the K8V4 layout of the pool's V)."""
    c = codes.astype(np.int16) & 15
    return (c[..., 0::2] | (c[..., 1::2] << 4)).astype(np.uint8).view(np.int8)


def make_pool(rng, n_kv, capacity, n_valid, d, poison=True, v_bits=8):
    """Draw one pool's valid cells in the fixed order K codes, K scales, V codes, V scales. v_bits = 4 (K8V4) draws
    V codes uniform on [-7, 7] and packs two per byte; the K side is the same as for v_bits = 8."""
    assert d % GROUP == 0 and 0 <= n_valid <= capacity and v_bits in (4, 8)
    ng = d // GROUP
    kc = _codes(rng, (n_kv, n_valid, d))
    ksc = _scales(rng, (n_kv, n_valid, ng))
    vc = _codes(rng, (n_kv, n_valid, d)) if v_bits == 8 else rng.integers(-7, 8, (n_kv, n_valid, d)).astype(np.int8)
    vsc = _scales(rng, (n_kv, n_valid, ng))
    fill_code = POISON_CODE if poison else 0
    fill_scale = np.float32(np.nan) if poison else np.float32(0)
    k = np.full((n_kv, capacity, d), fill_code, dtype=np.int8)
    ks = np.full((n_kv, capacity, ng), fill_scale, dtype=np.float32)
    vs = np.full((n_kv, capacity, ng), fill_scale, dtype=np.float32)
    k[:, :n_valid] = kc
    ks[:, :n_valid] = ksc
    vs[:, :n_valid] = vsc
    if v_bits == 8:
        v = np.full((n_kv, capacity, d), fill_code, dtype=np.int8)
        v[:, :n_valid] = vc
    else:   # poison: code -8 in both nibbles
        v = pack_v4(np.full((n_kv, capacity, d), -8 if poison else 0, dtype=np.int8))
        v[:, :n_valid] = pack_v4(vc)
    return Pool(k, ks, v, vs, capacity, n_valid, v_bits)


def make_q(rng, n_rows, n_q_heads, d):
    return (rng.standard_normal((n_rows, n_q_heads, d)) / math.sqrt(d)).astype(np.float32)


# name -> (n_slots, rows per slot, Hq, Hkv, d, capacity, n_valid, topk, n_chunks, bpc, n_active, prompt)
WORKLOADS = {
    # 1 query, 4/1 heads, 1,024 cells, top-8 of 16 blocks, 64-cell chunks.
    "tiny_decode": dict(slots=1, rows=1, hq=4, hkv=1, d=128, cap=1024, n_valid=1024, topk=8, n_chunks=8),
    # verify window: 4 queries at the last 4 positions of 16,384 valid cells, 200,000-cell capacity, top-32.
    "verify_window": dict(slots=1, rows=4, hq=24, hkv=4, d=128, cap=200_000, n_valid=16_384, topk=32,
                          n_chunks=20),
    # batch window: 2 slots x 2 rows, 65,536 valid cells per slot, top-64, one attention launch over both pools.
    "batch_window": dict(slots=2, rows=2, hq=24, hkv=4, d=128, cap=200_000, n_valid=65_536, topk=64,
                         n_chunks=20),
    # drafter: dense 32,768-cell window of 512 chunks of 64 cells, only the first 300 chunks populated.
    "drafter": dict(slots=1, rows=1, hq=24, hkv=4, d=128, cap=32_768, n_valid=19_200, topk=0, n_chunks=512,
                    bpc=1, n_active=300),
    # prompt chunk: 2,048 causal queries at the end of a 32,768-cell context.
    "prompt_chunk": dict(slots=1, rows=2048, hq=24, hkv=4, d=128, cap=32_768, n_valid=32_768, topk=0,
                         n_chunks=0, prompt=True),
}
WORKLOAD_ORDER = ["tiny_decode", "verify_window", "batch_window", "drafter", "prompt_chunk"]


def workload(name, poison=True, seed=None, **override):
    """Build a named workload. ``seed`` defaults to 1000 + its index in WORKLOAD_ORDER.

    Rows of a slot sit at the slot's last positions (a verify window is the newest cells of its context); the
    drafter's single query sees every populated cell; the prompt chunk's queries are the last rows of the context.
    ``override`` may shrink sizes (n_valid, cap, rows, ...) for fast parity cases.
    """
    spec = dict(WORKLOADS[name])
    spec.update(override)
    if seed is None:
        seed = 1000 + WORKLOAD_ORDER.index(name)
    rng = np.random.Generator(np.random.PCG64(seed))
    pools = [make_pool(rng, spec["hkv"], spec["cap"], spec["n_valid"], spec["d"], poison, spec.get("v_bits", 8))
             for _ in range(spec["slots"])]
    n_rows = spec["slots"] * spec["rows"]
    q = make_q(rng, n_rows, spec["hq"], spec["d"])
    pos = np.empty(n_rows, np.int32)
    row_pool = np.empty(n_rows, np.int32)
    for s in range(spec["slots"]):
        for r in range(spec["rows"]):
            pos[s * spec["rows"] + r] = spec["n_valid"] - spec["rows"] + r
            row_pool[s * spec["rows"] + r] = s
    prompt = spec.get("prompt", False)
    return Workload(name=name, n_q_heads=spec["hq"], n_kv_heads=spec["hkv"], head_dim=spec["d"], pools=pools,
                    q=q, pos=pos, row_pool=row_pool, topk=spec["topk"], n_chunks=spec["n_chunks"],
                    blocks_per_chunk=spec.get("bpc", 1), n_active=spec.get("n_active", 0), sm_scale=1.0,
                    prompt=prompt, pos0=int(pos[0]) if prompt else 0)


def random_pool(seed, n_kv, capacity, n_valid, d, poison=True, v_bits=8):
    rng = np.random.Generator(np.random.PCG64(seed))
    return make_pool(rng, n_kv, capacity, n_valid, d, poison, v_bits)


def random_q(seed, n_rows, n_q_heads, d):
    rng = np.random.Generator(np.random.PCG64(seed))
    return make_q(rng, n_rows, n_q_heads, d)


def random_scores(seed, n_rows, width, levels=0, p_ninf=0.0):
    """Score rows for top-k tests. ``levels`` > 0 draws from that many distinct values (tie-heavy rows);
    ``p_ninf`` marks that fraction of entries ineligible (-inf)."""
    rng = np.random.Generator(np.random.PCG64(seed))
    if levels > 0:
        s = rng.integers(0, levels, size=(n_rows, width)).astype(np.float32) - levels / 2
    else:
        s = rng.standard_normal((n_rows, width)).astype(np.float32)
    if p_ninf > 0:
        s[rng.random((n_rows, width)) < p_ninf] = -np.inf
    return s
