"""Benchmark of the QSA decode layer (block scores -> radix top-k -> split-K chunk attention -> LSE merge) on one
MI355X, plus the FP64 oracle timed on the host cores as a reported CPU baseline.

A step is one decode layer over one batch: the verify window (4 queries at the last 4 positions of 16,384 valid
cells in a 200,000-cell int8 pool, 24 q heads over 4 KV heads, head_dim 128, top-32 blocks of 64 cells per
(query, KV head)), run as one qsa_decode_layer call (fused block scores + top-k, chunk attention over 16 chunks,
merge). The block index is built beforehand (it is updated when cells are appended, not per query).
Inputs are resident in HBM before timing. Steps rotate over enough identical pool copies that the bytes they touch
exceed the 256 MB Infinity Cache, so K/V come from HBM; the layers are replayed from one captured HIP graph.

Prints one JSON line. `value` = algorithmic bytes of a layer / time per layer (GB/s); `roofline` reports the chunk
kernel (the dominant one): its algorithmic bytes per launch / its average launch duration, timed with HIP events
around graphs of back-to-back launches on the stream the kernels run on. The prompt chunk's roofline counts useful
ops (4 x head_dim per visible (query, q head, cell) pair) against the int8 peak; the digit-plane and issued int8
MFMA op counts are reported beside it under their own keys.
"""
from __future__ import annotations

import argparse
import json
import math
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0
INT8_PEAK_TOPS = 5000.0   # dense int8 matrix-core peak of an MI355X
BLOCK = 64
KV_BYTES_PER_CELL_HEAD = 128 + 128 + 8 + 8     # K and V codes plus their two fp32 group scales each, head_dim 128


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=1280)
    ap.add_argument("--warmup", type=int, default=128)
    ap.add_argument("--workload", default="verify_window",
                    choices=["tiny_decode", "verify_window", "drafter", "prompt_chunk"])
    ap.add_argument("--no-prompt", action="store_true", help="skip the prompt-chunk measurement")
    ap.add_argument("--no-other", action="store_true", help="skip the batch-window and drafter measurements")
    ap.add_argument("--prompt-steps", type=int, default=20)
    ap.add_argument("--v-bits", type=int, default=8, choices=[8, 4],
                    help="V format of the prompt chunk's pool with --workload prompt_chunk (4 = K8V4)")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run a plain device copy of known size (to scale HBM byte counters)")
    ap.add_argument("--copies", type=int, default=64, help="pool copies the steps rotate over")
    ap.add_argument("--chunks", type=int, default=0, help="split count (0 = the library default for the shape)")
    ap.add_argument("--pages-shapes", action="store_true",
                    help="time the shapes of the pages' own kernel tables and print them beside the pages' figures")
    ap.add_argument("--scale", action="store_true",
                    help="only measure the chunk kernel on 1, 2, 4 and 8 verify-window slots in one launch")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    return ap.parse_args()


def sources_hash(paths):
    """sha256 (first 16 hex digits) of the concatenated contents of the kernel's source files."""
    import hashlib
    h = hashlib.sha256()
    for rel in paths:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    return h.hexdigest()[:16]


def measured_traffic(key):
    """Per-launch HBM bytes (read + write) measured with rocprofv3 byte counters for this kernel's sources, or None
    once a source has changed since the counters were taken."""
    path = os.path.join(ROOT, "profiles", "traffic.json")
    if not os.path.exists(path):
        return None
    with open(path) as f:
        entry = json.load(f).get(key)
    if not entry:
        return None
    srcs = entry.get("sources") or [entry.get("source")]
    try:
        if sources_hash(srcs) != entry["sha256_16"]:
            return None
    except (OSError, TypeError, KeyError):
        return None
    return int(entry["read_bytes"] + entry["write_bytes"])


def measured_hbm_gbs(nbytes=1 << 30, reps=10):
    """HBM bandwidth a plain device-to-device copy reaches on this GPU (bytes read + written per second): the
    measured peak printed beside the datasheet's."""
    import torch
    src = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    dst = torch.empty_like(src)
    dst.copy_(src)
    torch.cuda.synchronize()
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record()
    for _ in range(reps):
        dst.copy_(src)
    b.record()
    torch.cuda.synchronize()
    gbs = 2 * nbytes * reps / (a.elapsed_time(b) * 1e-3) / 1e9
    del src, dst
    torch.cuda.empty_cache()
    return round(gbs, 1)


def union_cells(ids, counts, pos, n_valid, n_kv):
    """Number of distinct visible (KV head, cell) pairs the selected blocks of all rows touch."""
    n = 0
    for g in range(n_kv):
        cells = set()
        for i in range(ids.shape[0]):
            lim = min(int(pos[i]), n_valid - 1)
            for b in ids[i, g, :counts[i, g]]:
                if b < 0:
                    continue
                lo = int(b) * BLOCK
                hi = min(lo + BLOCK - 1, lim)
                if hi >= lo:
                    cells.update(range(lo, hi + 1))
        n += len(cells)
    return n


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print("bench.py measures one GPU: the QSA path here is single-GPU (sharding by KV head, slot or sequence is "
              "described in the design notes, not built); run with --gpus 1", file=sys.stderr)
        sys.exit(2)
    if args.copy_calibration:
        print(json.dumps(copy_calibration()))
        return
    if args.scale:
        for line in bench_scale():
            print(json.dumps(line), flush=True)
        return
    if args.pages_shapes:
        for line in bench_pages_shapes(args):
            print(json.dumps(line), flush=True)
        return
    if args.workload == "prompt_chunk":
        res = bench_prompt(args, args.steps if args.steps != 1280 else args.prompt_steps, main_line=True,
                           v_bits=args.v_bits)
    else:
        res = bench_decode(args)
        if args.workload == "verify_window" and not args.no_other:
            res["other_decode_workloads"] = bench_other_decode()
            res["pages_shapes"] = bench_pages_shapes(args)
        if not args.no_prompt:
            res["prompt_chunk"] = bench_prompt(args, args.prompt_steps, main_line=False)
            res["prompt_chunk_k8v4"] = bench_prompt(args, args.prompt_steps, main_line=False, v_bits=4, cpu=False)
    print(json.dumps(res))


def bench_decode(args):
    import torch

    import sparse_top_attention_amd as qsa
    import synth

    torch.cuda.set_device(0)
    dev = torch.device("cuda:0")
    w = synth.workload(args.workload, poison=False)
    pool_np = w.pools[0]
    dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
    n_rows, n_kv, D = w.q.shape[0], w.n_kv_heads, w.head_dim
    dense = w.topk == 0
    nb = -(-pool_np.n_valid // BLOCK)
    S = args.chunks or (w.n_chunks if dense else 16)   # sparse: 2 blocks (4 pieces of 32 cells) per chunk

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    # ---- inputs resident in HBM: one pool, then identical copies to rotate over
    base = qsa.Pool(t(pool_np.k), t(pool_np.ks), t(pool_np.v), t(pool_np.vs), pool_np.n_valid)
    base.index = torch.zeros(n_kv, -(-pool_np.capacity // BLOCK), D, dtype=torch.float32, device=dev)
    qsa.qsa_block_index(base, dims, 0, pool_np.n_valid, base.index)
    copies = [base]
    for _ in range(args.copies - 1):
        c = qsa.Pool(base.k.clone(), base.k_scale.clone(), base.v.clone(), base.v_scale.clone(), base.n_valid,
                     base.index.clone())
        copies.append(c)
    q = t(w.q)
    pos = t(w.pos)
    scores = torch.empty(n_rows, n_kv, max(nb, 1), dtype=torch.float32, device=dev)
    k = max(w.topk, 1)
    ids = torch.empty(n_rows, n_kv, k, dtype=torch.int32, device=dev)
    counts = torch.empty(n_rows, n_kv, dtype=torch.int32, device=dev)
    part = qsa.Partials.empty_like_shape(n_rows, w.n_q_heads, S, D, device=dev)
    # sized for the capacity-wide score rows too (the widest call below)
    layer_scratch = None if dense else torch.empty(
        qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, -(-pool_np.capacity // BLOCK), k, S), dtype=torch.uint8,
        device=dev)
    out = torch.empty(n_rows, w.n_q_heads, D, dtype=torch.float32, device=dev)
    lse = torch.empty(n_rows, w.n_q_heads, dtype=torch.float32, device=dev)
    n_active = t(np.full(n_rows, w.n_active, np.int32)) if dense else None
    torch.cuda.synchronize()

    def select(p):
        qsa.qsa_block_scores(q, pos, p, dims, nb, scores)
        qsa.qsa_topk(scores, w.topk, ids, counts)

    def attend(p):
        if dense:
            qsa.qsa_attn_chunk(q, pos, [p], dims, part, S, w.sm_scale, blocks_per_chunk=w.blocks_per_chunk)
        else:
            qsa.qsa_attn_chunk(q, pos, [p], dims, part, S, w.sm_scale, ids=ids, counts=counts)

    def merge():
        qsa.qsa_attn_merge(part, dims, S, out, lse, n_active=n_active)

    def layer_separate(p):
        if not dense:
            select(p)
        attend(p)
        merge()

    def fused_select(p):
        qsa.qsa_decode_select(q, pos, [p], dims, nb, w.topk, ids, counts)

    def fused_layer(p):
        qsa.qsa_decode_layer(q, pos, [p], dims, nb, w.topk, S, out, lse, sm_scale=w.sm_scale, ids=ids, counts=counts,
                             scratch=layer_scratch)

    # sparse workloads run the layer call (fused select launch, chunk launch, merge launch); the dense drafter call
    # has no selection and runs the chunk and active-merge calls
    layer = layer_separate if dense else fused_layer

    stream = torch.cuda.Stream()

    def capture(fn_per_copy, n, pools=None):
        pools = pools or copies
        g = torch.cuda.CUDAGraph()
        with torch.cuda.stream(stream):
            for c in range(n):               # eager pass so every kernel is loaded before capture
                fn_per_copy(pools[c % len(pools)])
        torch.cuda.synchronize()
        with torch.cuda.graph(g, stream=stream):
            for c in range(n):
                fn_per_copy(pools[c % len(pools)])
        torch.cuda.synchronize()
        return g

    L = len(copies)
    g_full = capture(layer, L)
    rem = args.steps % L
    g_rem = capture(layer, rem) if rem else None

    def run_steps(n_steps):
        for _ in range(n_steps // L):
            g_full.replay()
        if n_steps % L:
            (g_rem if n_steps % L == rem else capture(layer, n_steps % L)).replay()

    with torch.cuda.stream(stream):
        run_steps(args.warmup)
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        run_steps(args.steps)
        e1.record(stream)
        torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_per_step = ms_total / args.steps
    hbm_gbs = measured_hbm_gbs()

    # ---- per-kernel average launch durations: graphs of L back-to-back launches of one kernel, one per copy
    def kernel_avg_us(fn_per_copy, reps=20, pools=None):
        g = capture(fn_per_copy, L, pools)
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * L)

    # each call alone, back to back over the pool copies: the one-launch selection of qsa_decode_select (the layer
    # itself writes score rows in one launch and takes the top-k inside its chunk launch for rows of up to 1,024
    # blocks), the chunk kernel from given ids (the roofline's kernel) and the merge
    breakdown = {}
    separate = None
    if not dense:
        breakdown["select"] = kernel_avg_us(fused_select)
    breakdown["attn_chunk"] = kernel_avg_us(attend)
    breakdown["attn_merge"] = kernel_avg_us(lambda p: merge())
    capacity_wide = None
    if not dense:
        t_sep = kernel_avg_us(layer_separate)
        separate = {"us_per_layer": round(t_sep, 3), "block_scores+topk_us": round(kernel_avg_us(select), 3)}
        # capacity-wide selection: score rows over every block of the capacity (-inf past n_valid)
        nb_cap = -(-pool_np.capacity // BLOCK)

        def wide_select(p):
            qsa.qsa_decode_select(q, pos, [p], dims, nb_cap, w.topk, ids, counts)

        def wide_layer(p):
            qsa.qsa_decode_layer(q, pos, [p], dims, nb_cap, w.topk, S, out, lse, sm_scale=w.sm_scale, ids=ids,
                                 counts=counts, scratch=layer_scratch)
        capacity_wide = {"score_columns": nb_cap, "us_per_layer": round(kernel_avg_us(wide_layer), 3),
                         "select_us": round(kernel_avg_us(wide_select), 3)}
        # append path: the window's rows encode their new K/V cells (at their own positions) and refresh the index
        rng = np.random.default_rng(77)
        k_new = t(rng.standard_normal((n_rows, n_kv, D)).astype(np.float32))
        v_new = t(rng.standard_normal((n_rows, n_kv, D)).astype(np.float32))
        breakdown["kv_append"] = kernel_avg_us(lambda p: qsa.qsa_kv_append([p], dims, k_new, v_new, pos))
    chunk_key = "attn_chunk"
    k8v4 = None
    if not dense and D >= 128:
        # the same workload in K8V4 (4-bit V): its K side draws the same numbers, so the selection is the same
        k8v4 = bench_k8v4(args, w, dims, nb, S, q, pos, ids, counts, layer_scratch, out, lse, part,
                          lambda fn, pools: kernel_avg_us(fn, pools=pools), L)

    # ---- algorithmic bytes
    ids_h, counts_h = ids.cpu().numpy(), counts.cpu().numpy()
    if dense:
        vis = sum(min(pool_np.n_valid, int(p) + 1) for p in w.pos) * n_kv   # one row here
        kv_cells = vis
    else:
        kv_cells = union_cells(ids_h, counts_h, w.pos, pool_np.n_valid, n_kv)
    kv_bytes = kv_cells * KV_BYTES_PER_CELL_HEAD
    q_bytes = w.q.nbytes
    out_bytes = n_rows * w.n_q_heads * D * 4
    index_bytes = 0 if dense else n_kv * nb * D * 4
    layer_bytes = index_bytes + q_bytes + kv_bytes + out_bytes
    chunk_bytes = kv_bytes + q_bytes                       # what the chunk kernel must read, partials not counted
    chunk_gbs = chunk_bytes / (breakdown[chunk_key] * 1e-6) / 1e9
    value = layer_bytes / (ms_per_step * 1e-3) / 1e9

    result = {
        "metric": "decode QSA us/layer + HBM GB/s; prompt-chunk ms + int8 MFMA % of peak",
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 6),
        "us_per_layer": round(ms_per_step * 1e3, 3),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "f32",
        "data": "synthetic",
        "config": {"workload": args.workload, "rows": n_rows, "q_heads": w.n_q_heads, "kv_heads": n_kv,
                   "head_dim": D, "n_valid": pool_np.n_valid, "capacity": pool_np.capacity,
                   "topk_blocks": w.topk, "chunks": S, "pool_copies": L, "kv_int8": True,
                   "layer_bytes": int(layer_bytes), "kv_union_cells": int(kv_cells)},
        "kernels_us": {k2: round(v2, 3) for k2, v2 in breakdown.items()},
        "four_call_layer": separate,
        "capacity_wide": capacity_wide,
        "k8v4": k8v4,
        "roofline": {"bound": "hbm", "kernel": chunk_key, "achieved": round(chunk_gbs, 1),
                     "peak": HBM_PEAK_GBS, "unit": "GB/s", "frac": round(chunk_gbs / HBM_PEAK_GBS, 4),
                     "bytes_per_launch": int(chunk_bytes),
                     "traffic": measured_traffic(f"{chunk_key}_{args.workload}") if args.chunks == 0 else None,
                     "measured_peak": hbm_gbs, "frac_of_measured_peak": round(chunk_gbs / hbm_gbs, 4)},
        "cpu_baseline": None,
    }

    if not args.no_cpu_baseline:
        result["cpu_baseline"] = cpu_baseline(w, layer_bytes, args.cpu_seconds)
    del copies
    torch.cuda.empty_cache()
    return result


def bench_k8v4(args, w, dims, nb, S, q, pos, ids, counts, layer_scratch, out, lse, part, kernel_avg_us, L):
    """Layer and chunk-kernel times of the workload over K8V4 pool copies (int8 K, 4-bit V): K/V bytes per
    (cell, KV head) drop from 272 to 208 at head_dim 128."""
    import torch

    import sparse_top_attention_amd as qsa
    import synth

    dev = q.device
    p4 = synth.workload(args.workload, poison=False, v_bits=4).pools[0]

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)
    base = qsa.Pool(t(p4.k), t(p4.ks), t(p4.v), t(p4.vs), p4.n_valid, v_bits=4)
    base.index = torch.zeros(dims.n_kv_heads, -(-p4.capacity // BLOCK), dims.head_dim, dtype=torch.float32,
                             device=dev)
    qsa.qsa_block_index(base, dims, 0, p4.n_valid, base.index)
    pools = [base] + [qsa.Pool(base.k.clone(), base.k_scale.clone(), base.v.clone(), base.v_scale.clone(),
                               base.n_valid, base.index.clone(), v_bits=4) for _ in range(L - 1)]

    def layer(p):
        qsa.qsa_decode_layer(q, pos, [p], dims, nb, w.topk, S, out, lse, sm_scale=w.sm_scale, ids=ids, counts=counts,
                             scratch=layer_scratch)

    def attend(p):
        qsa.qsa_attn_chunk(q, pos, [p], dims, part, S, w.sm_scale, ids=ids, counts=counts)
    t_layer = kernel_avg_us(layer, pools)
    t_chunk = kernel_avg_us(attend, pools)
    ng = dims.head_dim // 64
    per_cell = dims.head_dim + 4 * ng + dims.head_dim // 2 + 4 * ng
    kv_cells = union_cells(ids.cpu().numpy(), counts.cpu().numpy(), w.pos, p4.n_valid, dims.n_kv_heads)
    chunk_bytes = kv_cells * per_cell + w.q.nbytes
    del pools
    return {"us_per_layer": round(t_layer, 3), "attn_chunk_us": round(t_chunk, 3), "kv_bytes_per_cell_head": per_cell,
            "attn_chunk_GBs": round(chunk_bytes / (t_chunk * 1e-6) / 1e9, 1)}


def bench_other_decode(copies=32, bw_chunks=32):
    """The batch window (2 slots x 2 rows, 65,536 valid cells per slot, top-64, one layer call over both pools) and
    the drafter (dense attention over 300 active 64-cell chunks of a 512-chunk window, active-only merge): per-call
    times and the chunk kernel's algorithmic bytes per launch over its time, against HBM peak. Pool copies rotate
    so K/V come from HBM."""
    import torch

    import sparse_top_attention_amd as qsa
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def avg_us(fn, n, reps=10):
        with torch.cuda.stream(stream):
            for c in range(n):
                fn(c)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in range(n):
                fn(c)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * n)

    def dev_pool(pn, with_index, dims):
        p = qsa.Pool(t(pn.k), t(pn.ks), t(pn.v), t(pn.vs), pn.n_valid)
        if with_index:
            p.index = torch.zeros(dims.n_kv_heads, -(-pn.capacity // BLOCK), dims.head_dim, dtype=torch.float32,
                                  device=dev)
            qsa.qsa_block_index(p, dims, 0, pn.n_valid, p.index)
        return p

    def clone(p):
        return qsa.Pool(p.k.clone(), p.k_scale.clone(), p.v.clone(), p.v_scale.clone(), p.n_valid,
                        None if p.index is None else p.index.clone())

    res = {}
    # ---- batch window
    w = synth.workload("batch_window", poison=False)
    dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
    n_rows, n_kv, D = w.q.shape[0], w.n_kv_heads, w.head_dim
    base = [dev_pool(pn, True, dims) for pn in w.pools]
    sets = [base] + [[clone(p) for p in base] for _ in range(copies - 1)]
    nb = -(-w.pools[0].n_valid // BLOCK)
    S = bw_chunks
    q, pos, row_pool = t(w.q), t(w.pos), t(w.row_pool)
    ids = torch.empty(n_rows, n_kv, w.topk, dtype=torch.int32, device=dev)
    counts = torch.empty(n_rows, n_kv, dtype=torch.int32, device=dev)
    out = torch.empty(n_rows, w.n_q_heads, D, dtype=torch.float32, device=dev)
    lse = torch.empty(n_rows, w.n_q_heads, dtype=torch.float32, device=dev)
    scratch = torch.empty(qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, nb, w.topk, S), dtype=torch.uint8,
                          device=dev)
    part = qsa.Partials.empty_like_shape(n_rows, w.n_q_heads, S, D, device=dev)

    def layer(c):
        qsa.qsa_decode_layer(q, pos, sets[c], dims, nb, w.topk, S, out, lse, sm_scale=w.sm_scale, row_pool=row_pool,
                             ids=ids, counts=counts, scratch=scratch)

    def chunk(c):
        qsa.qsa_attn_chunk(q, pos, sets[c], dims, part, S, w.sm_scale, row_pool=row_pool, ids=ids, counts=counts)

    # the layer's selection: with rows this wide it is the score launch then the top-k launch over a score buffer
    sel_scores = torch.empty(n_rows, n_kv, nb, dtype=torch.float32, device=dev)

    def select(c):
        qsa.qsa_decode_select(q, pos, sets[c], dims, nb, w.topk, ids, counts, scores=sel_scores, row_pool=row_pool)
    t_select = avg_us(select, copies)
    t_layer = avg_us(layer, copies)
    t_chunk = avg_us(chunk, copies)
    ids_h, counts_h = ids.cpu().numpy(), counts.cpu().numpy()
    cells = 0
    for sidx in range(len(w.pools)):
        rows = w.row_pool == sidx
        cells += union_cells(ids_h[rows], counts_h[rows], w.pos[rows], w.pools[sidx].n_valid, n_kv)
    cb = cells * KV_BYTES_PER_CELL_HEAD + w.q.nbytes
    gbs = cb / (t_chunk * 1e-6) / 1e9
    res["batch_window"] = {"us_per_layer": round(t_layer, 3), "select_us": round(t_select, 3),
                           "attn_chunk_us": round(t_chunk, 3),
                           "chunk_bytes_per_launch": int(cb), "attn_chunk_GBs": round(gbs, 1),
                           "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4), "chunks": S}
    del sets, base
    torch.cuda.empty_cache()

    # ---- drafter
    w = synth.workload("drafter", poison=False)
    dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
    pn = w.pools[0]
    base = dev_pool(pn, False, dims)
    pools = [base] + [clone(base) for _ in range(copies - 1)]
    q, pos = t(w.q), t(w.pos)
    part = qsa.Partials.empty_like_shape(1, w.n_q_heads, w.n_chunks, w.head_dim, device=dev)
    out = torch.empty(1, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    lse = torch.empty(1, w.n_q_heads, dtype=torch.float32, device=dev)
    n_active = t(np.array([w.n_active], np.int32))

    def dchunk(c):
        qsa.qsa_attn_chunk(q, pos, [pools[c]], dims, part, w.n_chunks, w.sm_scale, blocks_per_chunk=w.blocks_per_chunk)

    def dlayer(c):
        dchunk(c)
        qsa.qsa_attn_merge(part, dims, w.n_chunks, out, lse, n_active=n_active)
    t_chunk = avg_us(dchunk, copies)
    t_layer = avg_us(dlayer, copies)
    vis = min(pn.n_valid, int(w.pos[0]) + 1) * w.n_kv_heads
    cb = vis * KV_BYTES_PER_CELL_HEAD + w.q.nbytes
    gbs = cb / (t_chunk * 1e-6) / 1e9
    res["drafter"] = {"us_per_call": round(t_layer, 3), "attn_chunk_us": round(t_chunk, 3),
                      "chunk_bytes_per_launch": int(cb), "attn_chunk_GBs": round(gbs, 1),
                      "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4), "chunks": w.n_chunks, "active": w.n_active}
    del pools, base
    torch.cuda.empty_cache()
    return res


def bench_scale(slot_counts=(1, 2, 4, 8), chunk_counts=(4, 16)):
    """The verify window repeated over 1-8 slots (4 rows each, one 16,384-cell pool per slot) in one layer call:
    the chunk kernel's algorithmic bytes over its time as the launch grows, for a few chunk counts. Pool copies
    rotate so that about 450 MB of selected K/V separates two reads of the same bytes (they come from HBM)."""
    import torch

    import sparse_top_attention_amd as qsa
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def avg_us(fn, n, reps=10):
        with torch.cuda.stream(stream):
            for c in range(n):
                fn(c)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g, stream=stream):
            for c in range(n):
                fn(c)
        torch.cuda.synchronize()
        with torch.cuda.stream(stream):
            g.replay()
            torch.cuda.synchronize()
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(reps):
                g.replay()
            b.record(stream)
            torch.cuda.synchronize()
        return a.elapsed_time(b) * 1e3 / (reps * n)

    out = []
    for slots in slot_counts:
        w = synth.workload("verify_window", poison=False, slots=slots)
        dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
        copies = max(2, 64 // slots)

        def dev_pool(pn):
            p = qsa.Pool(t(pn.k), t(pn.ks), t(pn.v), t(pn.vs), pn.n_valid)
            p.index = torch.zeros(dims.n_kv_heads, -(-pn.capacity // BLOCK), dims.head_dim, dtype=torch.float32,
                                  device=dev)
            qsa.qsa_block_index(p, dims, 0, pn.n_valid, p.index)
            return p
        base = [dev_pool(pn) for pn in w.pools]
        sets = [base] + [[qsa.Pool(p.k.clone(), p.k_scale.clone(), p.v.clone(), p.v_scale.clone(), p.n_valid,
                                   p.index.clone()) for p in base] for _ in range(copies - 1)]
        n_rows = w.q.shape[0]
        nb = -(-w.pools[0].n_valid // BLOCK)
        q, pos, rp = t(w.q), t(w.pos), t(w.row_pool)
        ids = torch.empty(n_rows, w.n_kv_heads, w.topk, dtype=torch.int32, device=dev)
        counts = torch.empty(n_rows, w.n_kv_heads, dtype=torch.int32, device=dev)
        out_t = torch.empty(n_rows, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
        lse = torch.empty(n_rows, w.n_q_heads, dtype=torch.float32, device=dev)
        qsa.qsa_decode_select(q, pos, sets[0], dims, nb, w.topk, ids, counts, row_pool=rp)
        torch.cuda.synchronize()
        ih, ch = ids.cpu().numpy(), counts.cpu().numpy()
        cells = sum(union_cells(ih[w.row_pool == s], ch[w.row_pool == s], w.pos[w.row_pool == s],
                                w.pools[s].n_valid, w.n_kv_heads) for s in range(slots))
        cb = cells * KV_BYTES_PER_CELL_HEAD + w.q.nbytes
        for S in chunk_counts:
            scratch = torch.empty(qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, nb, w.topk, S),
                                  dtype=torch.uint8, device=dev)
            part = qsa.Partials.empty_like_shape(n_rows, w.n_q_heads, S, w.head_dim, device=dev)

            def layer(c):
                qsa.qsa_decode_layer(q, pos, sets[c], dims, nb, w.topk, S, out_t, lse, sm_scale=w.sm_scale,
                                     row_pool=rp, ids=ids, counts=counts, scratch=scratch)

            def chunk(c):
                qsa.qsa_attn_chunk(q, pos, sets[c], dims, part, S, w.sm_scale, row_pool=rp, ids=ids, counts=counts)
            tl, tc = avg_us(layer, copies), avg_us(chunk, copies)
            gbs = cb / (tc * 1e-6) / 1e9
            out.append({"workload": "verify_window x slots", "slots": slots, "rows": n_rows, "chunks": S,
                        "layer_us": round(tl, 2), "attn_chunk_us": round(tc, 2), "chunk_bytes_per_launch": int(cb),
                        "attn_chunk_GBs": round(gbs, 1), "frac_of_hbm": round(gbs / HBM_PEAK_GBS, 4)})
        del sets, base
        torch.cuda.empty_cache()
    return out


# The pages' own kernel tables, as context beside this library's time on the same shapes (other hardware, other
# engines; not targets): "#2806 sycl: decode QSA selection and attention in fewer, shorter launches", Summary
# (kernel table: one Arc Pro B70, 24 q heads, int8 K/V, 200,000-cell capacity, graph replay, us at 1K / 16K / 64K of
# context, the optimised column), and "#1367 prompt attention: STRATA_PROMPT_ATTN_IMMA=1 - the int8-KV kernel on
# INT8 tensor cores", Measured (per launch on an RTX 5090, the int8 kernel's column).
PAGES_LAYER_US = {(1, 1024): 62.3, (1, 16384): 107.9, (1, 65536): 156.2,
                  (2, 1024): 78.3, (2, 16384): 138.2, (2, 65536): 205.0}   # (rows per slot, context): us per layer
PAGES_DRAFTER_US = {1024: 41.0, 16384: 157.2, 65536: 335.9}                # one row, 32K window: us per call
PAGES_PROMPT_MS = {(32768, 2048): 1.55, (1500, 1500): 0.40, (2100, 256): 0.26}   # (context, queries): ms per launch


def _graph_avg_us(stream, fn, n, reps=10):
    """Mean us per call of fn(0) .. fn(n - 1), captured once in a HIP graph on `stream` and replayed reps times."""
    import torch
    with torch.cuda.stream(stream):
        for c in range(n):
            fn(c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in range(n):
            fn(c)
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        for _ in range(reps):
            g.replay()
        b.record(stream)
        torch.cuda.synchronize()
    return a.elapsed_time(b) * 1e3 / (reps * n)


def bench_pages_shapes(args, copies=16):
    """This library on the shapes of the pages' kernel tables (readings where the pages leave a size open: 4 KV
    heads, head_dim 128, top-64 blocks (all 16 at 1K, where the pages select every cell), 32 chunks per row (16 at
    1K); the drafter's 32K window holds min(context,
    32,768) valid cells in 512 chunks of 64 with an active-only merge; the prompt's queries are the last rows of
    their context). One JSON line per shape with the pages' figure and hardware beside it."""
    import torch

    import sparse_top_attention_amd as qsa
    import synth

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream()

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    def dev_pool(pn, dims, with_index):
        p = qsa.Pool(t(pn.k), t(pn.ks), t(pn.v), t(pn.vs), pn.n_valid)
        if with_index:
            p.index = torch.zeros(dims.n_kv_heads, -(-pn.capacity // BLOCK), dims.head_dim, dtype=torch.float32,
                                  device=dev)
            qsa.qsa_block_index(p, dims, 0, pn.n_valid, p.index)
        return p

    def clone(p):
        return qsa.Pool(p.k.clone(), p.k_scale.clone(), p.v.clone(), p.v_scale.clone(), p.n_valid,
                        None if p.index is None else p.index.clone())

    lines = []
    for rows in (1, 2):
        for ctx in (1024, 16384, 65536):
            w = synth.workload("batch_window", poison=False, rows=rows, n_valid=ctx, topk=min(64, -(-ctx // BLOCK)))
            dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
            base = [dev_pool(pn, dims, True) for pn in w.pools]
            sets = [base] + [[clone(p) for p in base] for _ in range(copies - 1)]
            n_rows, nb, S = w.q.shape[0], -(-ctx // BLOCK), 16 if ctx <= 1024 else 32
            q, pos, rp = t(w.q), t(w.pos), t(w.row_pool)
            ids = torch.empty(n_rows, w.n_kv_heads, w.topk, dtype=torch.int32, device=dev)
            counts = torch.empty(n_rows, w.n_kv_heads, dtype=torch.int32, device=dev)
            out = torch.empty(n_rows, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
            lse = torch.empty(n_rows, w.n_q_heads, dtype=torch.float32, device=dev)
            scratch = torch.empty(qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, nb, w.topk, S), dtype=torch.uint8,
                                  device=dev)

            def layer(c):
                qsa.qsa_decode_layer(q, pos, sets[c], dims, nb, w.topk, S, out, lse, sm_scale=w.sm_scale,
                                     row_pool=rp, ids=ids, counts=counts, scratch=scratch)
            us = _graph_avg_us(stream, layer, copies)
            lines.append({"shape": f"selection + attention per layer, 2 slots x {rows} row(s), {ctx} valid cells",
                          "us": round(us, 2), "pages_us": PAGES_LAYER_US[(rows, ctx)], "pages_hw": "Arc Pro B70",
                          "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "topk": w.topk, "chunks": S})
            del sets, base
            torch.cuda.empty_cache()
    for ctx in (1024, 16384, 65536):
        n_valid = min(ctx, 32768)
        w = synth.workload("drafter", poison=False, n_valid=n_valid, n_active=-(-n_valid // BLOCK))
        dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
        base = dev_pool(w.pools[0], dims, False)
        pools = [base] + [clone(base) for _ in range(copies - 1)]
        q, pos = t(w.q), t(w.pos)
        part = qsa.Partials.empty_like_shape(1, w.n_q_heads, w.n_chunks, w.head_dim, device=dev)
        out = torch.empty(1, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
        lse = torch.empty(1, w.n_q_heads, dtype=torch.float32, device=dev)
        n_active = t(np.array([w.n_active], np.int32))

        def drafter(c):
            qsa.qsa_attn_chunk(q, pos, [pools[c]], dims, part, w.n_chunks, w.sm_scale,
                               blocks_per_chunk=w.blocks_per_chunk)
            qsa.qsa_attn_merge(part, dims, w.n_chunks, out, lse, n_active=n_active)
        us = _graph_avg_us(stream, drafter, copies)
        lines.append({"shape": f"drafter call, one row, 32K window, {ctx} of context ({n_valid} valid cells, "
                               f"{w.n_active} active chunks)", "us": round(us, 2), "pages_us": PAGES_DRAFTER_US[ctx],
                      "pages_hw": "Arc Pro B70"})
        del pools, base
        torch.cuda.empty_cache()
    for (ctx, n_q), ms in PAGES_PROMPT_MS.items():
        r = bench_prompt(args, 16, main_line=False, cpu=False, shape=dict(n_valid=ctx, cap=ctx, rows=n_q))
        lines.append({"shape": f"prompt chunk, {n_q} queries at the end of a {ctx}-cell context",
                      "ms": r["ms_per_call"], "pages_ms": ms, "pages_hw": "RTX 5090",
                      "useful_int8_frac": r["roofline"]["frac"]})
    return lines


def copy_calibration(nbytes=1 << 28, reps=4):
    """A plain device-to-device copy of nbytes, reps times: a profiler's byte counters for these dispatches, divided
    by nbytes read and nbytes written, give the factor that turns counter readings into bytes."""
    import torch
    src = torch.ones(nbytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    torch.cuda.synchronize()
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    return {"copy_bytes_read": nbytes, "copy_bytes_written": nbytes, "reps": reps}


def prompt_ops(w):
    """Ops of one prompt chunk, per visible (query, q head, cell) pair:
    useful   -- the attention itself: d multiply-adds for q.k and d for p.v, 2 ops each (4 d per pair);
    planes   -- the same products on the pages' three 8-bit digit planes each (12 d per pair), the int8 work the
                pages' 24-bit split method implies;
    issued   -- the int8 MFMA ops the kernel actually issues: per 64-row block of a KV head and per 64-cell tile up
                to the block's last visible cell, 4 waves x (24 + 32) v_mfma_i32_16x16x64_i8 of 16*16*64*2 ops
                (3 q digit planes x 2 groups x 4 cell blocks for S^T, 4 p.w digit planes x 8 dim tiles for O^T);
                masked cells and padding rows included."""
    n_valid = w.pools[0].n_valid
    vis = sum(min(n_valid, int(p) + 1) for p in w.pos)
    pairs = vis * w.n_q_heads
    G = w.n_q_heads // w.n_kv_heads
    R = len(w.pos) * G
    tiles = 0
    for rb in range(-(-R // 64)):
        rlast = min(rb * 64 + 63, R - 1)
        c_end = min(n_valid, w.pos0 + rlast // G + 1)
        tiles += -(-c_end // 64)
    issued = tiles * w.n_kv_heads * 4 * (24 + 32) * 16 * 16 * 64 * 2
    return {"useful": pairs * w.head_dim * 4, "planes": pairs * w.head_dim * 12, "issued": issued}, vis


def bench_prompt(args, steps, main_line, v_bits=8, cpu=True, shape=None):
    """The 2,048-query prompt chunk at the end of a 32,768-cell context: one qsa_prompt_attn call per step, replayed
    from a HIP graph over pool copies (K/V and q are resident in HBM). v_bits 4 times a K8V4 pool of the same
    shape (same q and K draws, 4-bit V codes); `shape` overrides the workload's sizes (n_valid, cap, rows)."""
    import torch

    import sparse_top_attention_amd as qsa
    import synth

    dev = torch.device("cuda:0")
    w = synth.workload("prompt_chunk", poison=False, v_bits=v_bits, **(shape or {}))
    pool_np = w.pools[0]
    dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
    n_q = w.q.shape[0]
    tkey = "prompt_attn_prompt_chunk" + ("" if v_bits == 8 else "_k8v4")

    def t(a):
        return torch.from_numpy(np.ascontiguousarray(a)).to(dev)

    n_copies = 8
    base = qsa.Pool(t(pool_np.k), t(pool_np.ks), t(pool_np.v), t(pool_np.vs), pool_np.n_valid, v_bits=v_bits)
    copies = [base] + [qsa.Pool(base.k.clone(), base.k_scale.clone(), base.v.clone(), base.v_scale.clone(),
                                base.n_valid, v_bits=v_bits) for _ in range(n_copies - 1)]
    qs = [t(w.q)] + [None] * (n_copies - 1)
    for c in range(1, n_copies):
        qs[c] = qs[0].clone()
    scratch = torch.empty(qsa.qsa_prompt_scratch_bytes(n_q, w.pos0, dims), dtype=torch.uint8, device=dev)
    out = torch.empty(n_q, w.n_q_heads, w.head_dim, dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream()

    def call(c):
        qsa.qsa_prompt_attn(qs[c], w.pos0, copies[c], dims, out, sm_scale=w.sm_scale, scratch=scratch)

    with torch.cuda.stream(stream):
        for c in range(n_copies):
            call(c)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g, stream=stream):
        for c in range(n_copies):
            call(c)
    torch.cuda.synchronize()
    reps = max(1, -(-steps // n_copies))
    with torch.cuda.stream(stream):
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(reps):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
    n_calls = reps * n_copies
    ms = e0.elapsed_time(e1) / n_calls
    opc, vis = prompt_ops(w)
    ops = opc["useful"]
    tops = ops / (ms * 1e-3) / 1e12

    def frac(n):
        return round(n / (ms * 1e-3) / 1e12 / INT8_PEAK_TOPS, 4)

    res = {
        "workload": "prompt_chunk", "queries": n_q, "pos0": w.pos0, "n_valid": pool_np.n_valid,
        "q_heads": w.n_q_heads, "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "v_bits": v_bits,
        "ms_per_call": round(ms, 4), "calls_timed": n_calls,
        "roofline": {"bound": "mfma", "kernel": "qsa_prompt_attn (q split + attention + chunk merge)",
                     "achieved": round(tops, 1), "peak": INT8_PEAK_TOPS, "unit": "TOPS",
                     "frac": round(tops / INT8_PEAK_TOPS, 4), "ops_per_launch": int(ops),
                     "ops": "useful: 4 x head_dim per visible (query, q head, cell) pair (q.k and p.v)",
                     "traffic": measured_traffic(tkey)},
        "digit_plane_ops": {"ops_per_call": int(opc["planes"]), "frac_of_int8_peak": frac(opc["planes"]),
                            "about": "the useful products on three 8-bit digit planes each (the pages' 24-bit "
                                     "split): 3x the useful ops"},
        "issued_int8_mfma_ops": {"ops_per_call": int(opc["issued"]), "frac_of_int8_peak": frac(opc["issued"]),
                                 "about": "int8 MFMA ops the kernel issues (3 q planes + 4 p.w planes, whole "
                                          "64-cell tiles, padded rows): the matrix cores' busy share"},
    }
    if main_line:
        res = {
            "metric": "decode QSA us/layer + HBM GB/s; prompt-chunk ms + int8 MFMA % of peak",
            "value": round(tops, 2), "unit": "TOPS", "n_gpus": 1, "steps": n_calls, "warmup": n_copies,
            "ms_per_step": round(ms, 4), "higher_is_better": True, "scaling": "weak", "vs_baseline": None,
            "dtype": "i8", "data": "synthetic",
            "config": {"workload": "prompt_chunk", "queries": n_q, "q_heads": w.n_q_heads,
                       "kv_heads": w.n_kv_heads, "head_dim": w.head_dim, "n_valid": pool_np.n_valid,
                       "pos0": w.pos0, "v_bits": v_bits, "pool_copies": n_copies},
            "roofline": res["roofline"], "cpu_baseline": None}
    if cpu and not args.no_cpu_baseline:
        res["cpu_baseline"] = cpu_baseline_prompt(w, ops, vis, args.cpu_seconds)
    del copies, qs, scratch
    torch.cuda.empty_cache()
    return res


def host_cpu_model():
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return None


class one_core:
    """Pins this process to one of its allowed cores while the oracle is timed (it is single-threaded), then
    restores the affinity; a no-op where affinity cannot be set."""
    def __enter__(self):
        self.saved = None
        try:
            self.saved = os.sched_getaffinity(0)
            os.sched_setaffinity(0, {min(self.saved)})
        except (AttributeError, OSError):
            self.saved = None
        return self

    def __exit__(self, *exc):
        if self.saved is not None:
            os.sched_setaffinity(0, self.saved)


def cpu_baseline(w, layer_bytes, budget_s):
    """The FP64 oracle (single thread) on the same workload: scores, top-k and attention of one layer, repeated
    for about budget_s seconds; reported in the bench's unit (algorithmic bytes per layer / time per layer)."""
    import oracle
    pool = w.pools[0]
    n_kv = w.n_kv_heads
    nb = -(-pool.n_valid // BLOCK)
    r = oracle.block_index(pool)          # append-time step, outside the timed sample as on the GPU
    dense = w.topk == 0
    n = 0
    with one_core():
        t0 = time.perf_counter()
        while True:
            if dense:
                oracle.attn(w.q, w.pos, pool, n_kv)
            else:
                s = oracle.block_scores(w.q, w.pos, r, n_kv, pool.n_valid, nb)
                ids, cnt = oracle.topk(s.reshape(-1, nb), w.topk)
                oracle.attn(w.q, w.pos, pool, n_kv, ids=ids.reshape(len(w.pos), n_kv, -1),
                            counts=cnt.reshape(len(w.pos), n_kv))
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    per_layer = el / n
    return {"value": round(layer_bytes / per_layer / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"{n} full {w.name} layers (scores, top-k, attention; FP64, one thread) in {el:.1f} s, "
                      f"{per_layer * 1e3:.1f} ms per layer, pinned to one core", "host_cpus": os.cpu_count(),
            "host_cpu": host_cpu_model()}


def cpu_baseline_prompt(w, ops, vis, budget_s):
    """The FP64 oracle on sampled (query, head) rows of the prompt chunk for about budget_s seconds, scaled to the
    whole chunk's algorithmic ops (rows differ only in their causal length)."""
    import oracle
    pool = w.pools[0]
    rng = np.random.default_rng(0)
    n_q = w.q.shape[0]
    done_cells, n = 0, 0
    with one_core():
        t0 = time.perf_counter()
        while True:
            i, h = int(rng.integers(0, n_q)), int(rng.integers(0, w.n_q_heads))
            oracle.attn_one(w.q, w.pos, i, h, pool, w.n_kv_heads)
            done_cells += min(pool.n_valid, int(w.pos[i]) + 1)
            n += 1
            el = time.perf_counter() - t0
            if el >= budget_s:
                break
    per_cell = el / done_cells
    full_s = per_cell * vis * w.n_q_heads
    return {"value": round(ops / full_s / 1e12, 6), "unit": "TOPS", "cores": 1, "kind": "oracle",
            "sample": f"{n} random (query, head) rows of the prompt chunk (FP64 dense attention, one thread) in "
                      f"{el:.1f} s; scaled to the chunk's {vis * w.n_q_heads} (row, cell) pairs: {full_s:.0f} s "
                      f"per chunk, pinned to one core", "host_cpus": os.cpu_count(), "host_cpu": host_cpu_model()}


if __name__ == "__main__":
    main()
