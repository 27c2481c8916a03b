"""Parity of the decode path on the GPU against the FP64 oracle, through the C ABI.

Bars: ids and counts bit-exact; empty marks bit-exact; outputs within a max relative error of 1e-5 per
(row, head) (max_d |x - y| / max_d |y|); scores within 1e-5 of sum_d |qsum_d r_d|. Pools carry poison (NaN
scales, codes -128) past n_valid and the block index is NaN-filled past the valid blocks, so a read outside the
valid cells shows up as a NaN or a mismatch.
"""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_attention_amd as qsa
import synth
from gpu_util import (BLOCK, build_index, decode_layer, dev, qsum_abs_dot, rel_err_rows, score_errors,
                      to_device, topk_margin_ok)

pytestmark = pytest.mark.gpu
TOL = 1e-5


def dims_of(w):
    return qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)


def small_workload(seed, n_kv=2, G=3, d=128, cap=1400, n_valid=1290, rows=3, topk=7, v_bits=8):
    pool = synth.random_pool(seed, n_kv, cap, n_valid, d, v_bits=v_bits)
    q = synth.random_q(seed + 1, rows, n_kv * G, d)
    pos = np.array([n_valid - rows + r for r in range(rows)], np.int32)
    return synth.Workload("small", n_kv * G, n_kv, d, [pool], q, pos, np.zeros(rows, np.int32), topk, 5, 1, 0, 1.0)


# ------------------------------------------------------------------------------------------------ index
@pytest.mark.parametrize("d,n_valid,cap", [(128, 1290, 1400), (64, 64, 64), (256, 700, 1000), (192, 1000, 1100),
                                           (128, 16384, 200_000)])
def test_block_index(d, n_valid, cap):
    pool = synth.random_pool(7, 2, cap, n_valid, d)
    dims = qsa.Dims(6, 2, d)
    p = build_index(to_device(pool), dims)
    torch.cuda.synchronize()
    nb = -(-n_valid // BLOCK)
    got = p.index.cpu().numpy()
    ref = oracle.block_index(pool)
    assert rel_err_rows(got[:, :nb], ref).max() <= TOL
    assert np.all(np.isnan(got[:, nb:]))          # blocks past n_valid untouched by a [0, n_valid) update


def test_block_index_partial_range_touches_only_its_blocks():
    pool = synth.random_pool(9, 2, 1000, 900, 128)
    dims = qsa.Dims(4, 2, 128)
    p = to_device(pool)
    qsa.qsa_block_index(p, dims, 130, 200, p.index)      # cells 130..199 -> blocks 2 and 3
    qsa.qsa_block_index(p, dims, 880, 1000, p.index)     # blocks 13 (partly valid) .. 15 (no valid cell)
    torch.cuda.synchronize()
    got = p.index.cpu().numpy()
    ref = oracle.block_index(pool, n_blocks=16)
    for b in range(16):
        if b in (2, 3, 13, 14, 15):
            assert rel_err_rows(got[:, b], ref[:, b]).max() <= TOL, b
        else:
            assert np.all(np.isnan(got[:, b])), b
    assert np.all(got[:, 15] == 0)


# ----------------------------------------------------------------------------------------------- scores
@pytest.mark.parametrize("d,G,rows", [(128, 6, 4), (64, 1, 1), (256, 8, 3), (128, 5, 9), (192, 3, 5)])
def test_block_scores(d, G, rows):
    n_kv, n_valid, cap = 2, 3000, 4096
    pool = synth.random_pool(11, n_kv, cap, n_valid, d)
    q = synth.random_q(12, rows, n_kv * G, d)
    pos = np.array([n_valid - 1 - 37 * r for r in range(rows)], np.int32)
    dims = qsa.Dims(n_kv * G, n_kv, d)
    p = build_index(to_device(pool), dims)
    nb = 60                                               # wider than ceil(n_valid/64) = 47
    s = torch.empty(rows, n_kv, nb, dtype=torch.float32, device="cuda")
    qsa.qsa_block_scores(dev(q), dev(pos), p, dims, nb, s)
    torch.cuda.synchronize()
    r32 = p.index.cpu().numpy()[:, :47].astype(np.float64)
    ref = oracle.block_scores(q, pos, r32, n_kv, n_valid, nb)
    scale = np.zeros_like(ref)
    scale[..., :47] = qsum_abs_dot(q, r32, G)
    err = score_errors(s.cpu().numpy().astype(np.float64), ref, scale)
    assert err.max() <= TOL


# ------------------------------------------------------------------------------------------------- top-k
@pytest.mark.parametrize("width,k,levels,p_ninf", [
    (16, 8, 0, 0.0), (256, 32, 0, 0.0), (1024, 64, 0, 0.0), (256, 32, 4, 0.0), (1000, 64, 3, 0.2),
    (3125, 64, 0, 0.0), (4096, 100, 2, 0.5), (16384, 64, 0, 0.0), (100, 100, 0, 0.3), (33, 1, 1, 0.0),
    (64, 5, 0, 1.0), (1, 1, 0, 0.0), (300, 299, 5, 0.0),
])
def test_topk_bit_exact(width, k, levels, p_ninf):
    rows = 17
    s = synth.random_scores(100 + width + k, rows, width, levels=levels, p_ninf=p_ninf)
    if width >= 8:
        s[0, :4] = -0.0
        s[0, 4:8] = 0.0
    ids = torch.empty(rows, k, dtype=torch.int32, device="cuda")
    counts = torch.empty(rows, dtype=torch.int32, device="cuda")
    qsa.qsa_topk(dev(s), k, ids, counts)
    torch.cuda.synchronize()
    ref_ids, ref_counts = oracle.topk(s.astype(np.float64), k)
    assert np.array_equal(ids.cpu().numpy(), ref_ids)
    assert np.array_equal(counts.cpu().numpy(), ref_counts)


# ---------------------------------------------------------------------------------------- chunk + merge
def _partials_vs_oracle(w, p_dev, dims, S, ids, counts, gpu_counts=None):
    q, pos = dev(w.q), dev(w.pos)
    part = qsa.Partials.empty_like_shape(w.q.shape[0], dims.n_q_heads, S + 2, dims.head_dim)
    gc = counts if gpu_counts is None else gpu_counts
    qsa.qsa_attn_chunk(q, pos, [p_dev], dims, part, S, w.sm_scale, ids=dev(ids), counts=dev(gc))
    torch.cuda.synchronize()
    gm, gl, go, ge = (t.cpu().numpy()[:, :, :S] for t in (part.m, part.l, part.o, part.empty))
    rm, rl, ro, re = oracle.chunk_partials(w.q, w.pos, w.pools[0], w.n_kv_heads, S, ids=ids, counts=counts)
    assert np.array_equal(ge, re)
    full = ~re.astype(bool)
    assert np.all(gm[~full] == -np.inf) and np.all(gl[~full] == 0) and np.all(go[~full] == 0)
    lse_g = gm[full].astype(np.float64) + np.log(gl[full].astype(np.float64))
    lse_r = rm[full] + np.log(rl[full])
    assert np.abs(lse_g - lse_r).max() <= TOL
    og = go[full] / gl[full][:, None]
    orr = ro[full] / rl[full][:, None]
    assert rel_err_rows(og, orr).max() <= TOL
    return part


@pytest.mark.parametrize("S", [1, 3, 5, 7, 12])
def test_chunk_partials(S):
    w = small_workload(21)
    dims = dims_of(w)
    pool = w.pools[0]
    nb = -(-pool.n_valid // BLOCK)
    s = oracle.block_scores(w.q, w.pos, oracle.block_index(pool), 2, pool.n_valid, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), w.topk)
    ids, counts = ids.reshape(3, 2, -1), counts.reshape(3, 2)
    _partials_vs_oracle(w, to_device(pool), dims, S, ids, counts)


@pytest.mark.parametrize("d", [128, 192])
def test_chunk_partials_short_selection_and_bad_ids(d):
    w = small_workload(23, rows=3, d=d)
    dims = dims_of(w)
    ids = np.array([[[0, 5, 19, -1, -1, -1, -1], [20, 3, 7, 8, 9, 1, 2]],      # row 0: 3 of 7 valid
                    [[-1] * 7, [4, 1 << 30, -7, 6, 100000, 2, 19]],           # row 1: none; junk ids skipped
                    [[19, 20, 0, 1, 2, 3, 4], [5, 6, 7, 8, 9, 10, 11]]], np.int32)
    counts = np.array([[3, 7], [0, 7], [7, 9]], np.int32)                      # 9 > k: the kernel clamps to 7
    _partials_vs_oracle(w, to_device(w.pools[0]), dims, 4, ids, np.minimum(counts, 7), gpu_counts=counts)
    neg = counts.copy()
    neg[0, 0] = -3                                                              # negative count: no block
    ref_counts = np.minimum(neg, 7).clip(min=0)
    _partials_vs_oracle(w, to_device(w.pools[0]), dims, 4, ids, ref_counts, gpu_counts=neg)


@pytest.mark.parametrize("d,G", [(64, 1), (64, 4), (64, 6), (64, 8), (128, 1), (128, 2), (128, 5), (128, 8),
                                 (192, 1), (192, 4), (192, 6), (192, 8), (256, 1), (256, 3), (256, 6), (256, 8)])
def test_decode_head_dims_and_group_sizes(d, G):
    w = small_workload(31 + d + G, n_kv=2, G=G, d=d, cap=2100, n_valid=2010, rows=2, topk=9)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    got = decode_layer(w, p, dims, n_chunks=4)
    _check_end_to_end(w, got)


def test_merge_active_and_garbage():
    """Chunks at or past n_active are not read even when unmarked and holding garbage."""
    w = small_workload(41)
    dims = dims_of(w)
    pool = w.pools[0]
    ids, counts = oracle.full_selection(w.pos, 2, pool.n_valid, 7)
    part = _partials_vs_oracle(w, to_device(pool), dims, 6, ids, counts)
    part.m[:, :, 6:] = 1e30
    part.l[:, :, 6:] = float("nan")
    part.o[:, :, 6:] = float("nan")
    part.empty[:, :, 6:] = 0
    n_active = torch.tensor([6, 6, 6], dtype=torch.int32, device="cuda")
    out = torch.empty(3, 6, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(3, 6, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, 8, out, lse, n_active=n_active)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attn(w.q, w.pos, pool, 2, ids=ids, counts=counts)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= TOL * np.abs(ref_lse).max()


@pytest.mark.parametrize("S,n_act", [(150, None), (97, np.array([97, 65, 3], np.int32))])
def test_merge_many_chunks_skips_empty_garbage(S, n_act):
    """More than 64 chunks (the merge's split-dims form, two chunks per row step): chunks marked empty hold NaN in
    m, l and o and change nothing; an odd number of active chunks leaves the last step's second chunk unused."""
    w = small_workload(47)
    pool = w.pools[0]
    dims = dims_of(w)
    m, l, o, e = oracle.chunk_partials(w.q, w.pos, pool, 2, S, bpc=1)
    assert e[:, :, 30:].all() and not e[:, :, :5].any()
    m32, l32, o32 = m.astype(np.float32), l.astype(np.float32), o.astype(np.float32)
    m32[e.astype(bool)] = np.nan
    l32[e.astype(bool)] = np.nan
    o32[e.astype(bool)] = np.nan
    part = qsa.Partials(dev(m32), dev(l32), dev(o32), dev(e))
    out = torch.empty(3, 6, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(3, 6, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, S, out, lse, n_active=None if n_act is None else dev(n_act))
    torch.cuda.synchronize()
    ref, ref_lse = oracle.merge(m, l, o, e, n_active=n_act)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= TOL * np.abs(ref_lse).max()


def test_merge_of_oracle_partials():
    """The merge alone, fed FP64-computed partials rounded to fp32."""
    w = small_workload(43)
    pool = w.pools[0]
    dims = dims_of(w)
    S = 9
    m, l, o, e = oracle.chunk_partials(w.q, w.pos, pool, 2, S, bpc=3)
    part = qsa.Partials(dev(m.astype(np.float32)), dev(l.astype(np.float32)), dev(o.astype(np.float32)), dev(e))
    for n_act in (None, np.array([9, 4, 0], np.int32)):
        out = torch.empty(3, 6, 128, dtype=torch.float32, device="cuda")
        lse = torch.empty(3, 6, dtype=torch.float32, device="cuda")
        qsa.qsa_attn_merge(part, dims, S, out, lse, n_active=None if n_act is None else dev(n_act))
        torch.cuda.synchronize()
        ref, ref_lse = oracle.merge(m, l, o, e, n_active=n_act)
        assert rel_err_rows(out.cpu().numpy(), ref).max() <= TOL
        fin = np.isfinite(ref_lse)
        assert np.array_equal(np.isneginf(lse.cpu().numpy()), ~fin)
        assert np.abs(lse.cpu().numpy()[fin] - ref_lse[fin]).max() <= TOL


def test_all_empty_rows_and_bad_pool_index():
    w = small_workload(45, rows=3)
    dims = dims_of(w)
    pool = w.pools[0]
    pos = w.pos.copy()
    pos[1] = -5                                         # sees no cell
    q, posd = dev(w.q), dev(pos)
    p = to_device(pool)
    row_pool = dev(np.array([0, 0, 3], np.int32))       # row 2 names a pool that does not exist
    part = qsa.Partials.empty_like_shape(3, 6, 4, 128)
    qsa.qsa_attn_chunk(q, posd, [p], dims, part, 4, 1.0, row_pool=row_pool, blocks_per_chunk=6)
    out = torch.empty(3, 6, 128, dtype=torch.float32, device="cuda")
    lse = torch.empty(3, 6, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, 4, out, lse)
    torch.cuda.synchronize()
    e = part.empty.cpu().numpy()
    assert np.all(e[1] == 1) and np.all(e[2] == 1) and np.all(e[0, :, :4] == 0)
    o = out.cpu().numpy()
    assert np.all(o[1:] == 0) and np.all(np.isneginf(lse.cpu().numpy()[1:]))
    ref, _ = oracle.attn(w.q[:1], w.pos[:1], pool, 2)
    assert rel_err_rows(o[:1], ref).max() <= TOL


# ------------------------------------------------------------------------------------------- end to end
def _check_end_to_end(w, got, pool=None, rows=None):
    pool = pool or w.pools[0]
    rows = slice(None) if rows is None else rows
    q, pos = w.q[rows], w.pos[rows]
    n_kv, G = w.n_kv_heads, w.n_q_heads // w.n_kv_heads
    nb = -(-pool.n_valid // BLOCK)
    r = oracle.block_index(pool)
    s_ref = oracle.block_scores(q, pos, r, n_kv, pool.n_valid, nb)
    # scores against the oracle's FP64 index
    scale = qsum_abs_dot(q, r, G)
    assert score_errors(got["scores"].astype(np.float64), s_ref, scale).max() <= TOL
    # ids: bit-exact against the FP64 selection, on rows whose k-th margin clears the fp32 error band
    ids_ref, cnt_ref = oracle.topk(s_ref.reshape(-1, nb), w.topk)
    ok = topk_margin_ok(s_ref.reshape(-1, nb), w.topk, scale.reshape(-1, nb))
    assert ok.all(), f"{(~ok).sum()} tie-ambiguous rows"
    assert np.array_equal(got["ids"].reshape(-1, w.topk), ids_ref)
    assert np.array_equal(got["counts"].reshape(-1), cnt_ref)
    # ids: bit-exact against the oracle's top-k of the GPU's own fp32 scores
    ids2, cnt2 = oracle.topk(got["scores"].astype(np.float64).reshape(-1, nb), w.topk)
    assert np.array_equal(got["ids"].reshape(-1, w.topk), ids2)
    # attention over the selected cells
    ref, ref_lse = oracle.attn(q, pos, pool, n_kv, ids=ids_ref.reshape(len(pos), n_kv, -1),
                               counts=cnt_ref.reshape(len(pos), n_kv))
    assert rel_err_rows(got["out"], ref).max() <= TOL
    assert np.abs(got["lse"] - ref_lse).max() <= TOL * max(1.0, np.abs(ref_lse).max())


@pytest.mark.parametrize("name,S", [("tiny_decode", 8), ("verify_window", 20), ("verify_window", 7),
                                    ("verify_window", 32)])
def test_end_to_end_single_pool(name, S):
    w = synth.workload(name)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    got = decode_layer(w, p, dims, n_chunks=S)
    _check_end_to_end(w, got)


def _batch_window_run(w, dims, S, multi=True):
    pdevs = [build_index(to_device(pl), dims) for pl in w.pools]
    n_rows = w.q.shape[0]
    q, pos = dev(w.q), dev(w.pos)
    nb = -(-w.pools[0].n_valid // BLOCK)
    scores = torch.empty(n_rows, dims.n_kv_heads, nb, dtype=torch.float32, device="cuda")
    for sidx, pd in enumerate(pdevs):                  # scores once per slot (a slot's rows are contiguous)
        rows = slice(2 * sidx, 2 * sidx + 2)
        qsa.qsa_block_scores(q[rows], pos[rows], pd, dims, nb, scores[rows])
    ids = torch.empty(n_rows, dims.n_kv_heads, w.topk, dtype=torch.int32, device="cuda")
    counts = torch.empty(n_rows, dims.n_kv_heads, dtype=torch.int32, device="cuda")
    qsa.qsa_topk(scores, w.topk, ids, counts)          # top-k once per window
    part = qsa.Partials.empty_like_shape(n_rows, dims.n_q_heads, S, dims.head_dim)
    if multi:                                         # attention once per window over both pools
        qsa.qsa_attn_chunk(q, pos, pdevs, dims, part, S, w.sm_scale, row_pool=dev(w.row_pool), ids=ids,
                           counts=counts)
    else:                                             # one call per slot
        for sidx, pd in enumerate(pdevs):
            rows = slice(2 * sidx, 2 * sidx + 2)
            sub = qsa.Partials(part.m[rows], part.l[rows], part.o[rows], part.empty[rows])
            qsa.qsa_attn_chunk(q[rows], pos[rows], [pd], dims, sub, S, w.sm_scale, ids=ids[rows].contiguous(),
                               counts=counts[rows].contiguous())
    out = torch.empty(n_rows, dims.n_q_heads, dims.head_dim, dtype=torch.float32, device="cuda")
    lse = torch.empty(n_rows, dims.n_q_heads, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, S, out, lse)
    torch.cuda.synchronize()
    return dict(scores=scores.cpu().numpy(), ids=ids.cpu().numpy(), counts=counts.cpu().numpy(),
                out=out.cpu().numpy(), lse=lse.cpu().numpy(), o=part.o.cpu().numpy())


def test_end_to_end_batch_window():
    w = synth.workload("batch_window")
    dims = dims_of(w)
    got = _batch_window_run(w, dims, S=20)
    for sidx in range(2):
        rows = slice(2 * sidx, 2 * sidx + 2)
        sub = {k: v[rows] for k, v in got.items()}
        _check_end_to_end(w, sub, pool=w.pools[sidx], rows=rows)


def test_multi_pool_equals_per_slot_calls():
    """One chunk launch over both slots' pools gives the bits of one launch per slot."""
    w = synth.workload("batch_window")
    dims = dims_of(w)
    a = _batch_window_run(w, dims, S=12, multi=True)
    b = _batch_window_run(w, dims, S=12, multi=False)
    assert np.array_equal(a["o"], b["o"]) and np.array_equal(a["out"], b["out"])


def test_end_to_end_drafter_dense_active_merge():
    w = synth.workload("drafter")
    dims = dims_of(w)
    pool = w.pools[0]
    p = to_device(pool)
    q, pos = dev(w.q), dev(w.pos)
    part = qsa.Partials.empty_like_shape(1, dims.n_q_heads, w.n_chunks, dims.head_dim)
    qsa.qsa_attn_chunk(q, pos, [p], dims, part, w.n_chunks, w.sm_scale, blocks_per_chunk=w.blocks_per_chunk)
    outs = []
    for n_act in (dev(np.array([w.n_active], np.int32)), None):
        out = torch.empty(1, dims.n_q_heads, dims.head_dim, dtype=torch.float32, device="cuda")
        lse = torch.empty(1, dims.n_q_heads, dtype=torch.float32, device="cuda")
        qsa.qsa_attn_merge(part, dims, w.n_chunks, out, lse, n_active=n_act)
        outs.append((out, lse))
    torch.cuda.synchronize()
    e = part.empty.cpu().numpy()
    assert np.all(e[..., :w.n_active] == 0) and np.all(e[..., w.n_active:] == 1)
    ref, ref_lse = oracle.attn(w.q, w.pos, pool, w.n_kv_heads)
    for out, lse in outs:
        assert rel_err_rows(out.cpu().numpy(), ref).max() <= TOL
        assert np.abs(lse.cpu().numpy() - ref_lse).max() <= TOL * np.abs(ref_lse).max()


def test_split_count_does_not_change_output():
    w = synth.workload("verify_window")
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    outs = [decode_layer(w, p, dims, n_chunks=S)["out"] for S in (1, 2, 5, 20, 32)]
    pool = w.pools[0]
    nb = -(-pool.n_valid // BLOCK)
    s_ref = oracle.block_scores(w.q, w.pos, oracle.block_index(pool), 4, pool.n_valid, nb)
    ids, cnt = oracle.topk(s_ref.reshape(-1, nb), w.topk)
    ref, _ = oracle.attn(w.q, w.pos, pool, 4, ids=ids.reshape(4, 4, -1), counts=cnt.reshape(4, 4))
    for o in outs:
        assert rel_err_rows(o, ref).max() <= TOL


def test_repeat_runs_are_bitwise_identical():
    w = synth.workload("verify_window")
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    a = decode_layer(w, p, dims, n_chunks=16)
    b = decode_layer(w, p, dims, n_chunks=16)
    for key in ("scores", "ids", "out", "lse", "m", "l", "o"):
        assert np.array_equal(a[key], b[key]), key


@pytest.mark.parametrize("n_chunks,rows", [(301, 2), (7, 3)])
def test_dense_partials_one_and_two_waves_per_chunk(n_chunks, rows):
    """Dense 64-cell chunks: with many chunks a wave walks a whole chunk (one wave per chunk, four chunks per
    workgroup, the last workgroup partly empty); with few, two waves share one. Partials against the oracle's."""
    cap = 64 * n_chunks + 100
    w = small_workload(61 + n_chunks, n_kv=2, G=3, cap=cap, n_valid=cap - 150, rows=rows, topk=4)
    dims = dims_of(w)
    q, pos = dev(w.q), dev(w.pos)
    part = qsa.Partials.empty_like_shape(rows, dims.n_q_heads, n_chunks + 1, dims.head_dim)
    qsa.qsa_attn_chunk(q, pos, [to_device(w.pools[0])], dims, part, n_chunks, w.sm_scale, blocks_per_chunk=1)
    torch.cuda.synchronize()
    gm, gl, go, ge = (t.cpu().numpy()[:, :, :n_chunks] for t in (part.m, part.l, part.o, part.empty))
    rm, rl, ro, re = oracle.chunk_partials(w.q, w.pos, w.pools[0], w.n_kv_heads, n_chunks, bpc=1)
    assert np.array_equal(ge, re)
    full = ~re.astype(bool)
    assert np.all(gm[~full] == -np.inf) and np.all(gl[~full] == 0) and np.all(go[~full] == 0)
    lse_g = gm[full].astype(np.float64) + np.log(gl[full].astype(np.float64))
    lse_r = rm[full] + np.log(rl[full])
    assert np.abs(lse_g - lse_r).max() <= TOL
    assert rel_err_rows(go[full] / gl[full][:, None], ro[full] / rl[full][:, None]).max() <= TOL


@pytest.mark.parametrize("G,v_bits,d", [(6, 8, 128), (2, 8, 128), (6, 4, 128), (6, 8, 192)],
                         ids=["mfma-int8", "valu-int8", "mfma-k8v4", "valu-int8-d192"])
@pytest.mark.parametrize("scale", [-0.7, 0.0, 3.0])
def test_dense_chunks_any_finite_scale(G, v_bits, d, scale):
    """sm_scale may be any finite value: a negative one flips which cells dominate, zero gives uniform weights over
    the visible cells, a large one sharpens the softmax. Dense chunks and the merge against the oracle."""
    w = small_workload(71 + G + v_bits, n_kv=2, G=G, d=d, cap=900, n_valid=830, rows=3, v_bits=v_bits)
    dims = dims_of(w)
    n_chunks = 4
    part = qsa.Partials.empty_like_shape(3, dims.n_q_heads, n_chunks, dims.head_dim)
    qsa.qsa_attn_chunk(dev(w.q), dev(w.pos), [to_device(w.pools[0])], dims, part, n_chunks, scale, blocks_per_chunk=4)
    out = torch.empty(3, dims.n_q_heads, dims.head_dim, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, n_chunks, out)
    torch.cuda.synchronize()
    ref, _ = oracle.attn(w.q, w.pos, w.pools[0], w.n_kv_heads, sm_scale=scale)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= TOL
