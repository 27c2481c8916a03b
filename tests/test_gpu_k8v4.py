"""Parity of the K8V4 pool format (int8 K, signed 4-bit V packed two per byte, per-64-dim scales) on the decode
path, through the C ABI: chunk partials, the three-launch layer (selected and dense) and the append encoder, against
the FP64 oracle reading the same packed bytes. K8V4 is a cache format the pages list beside int8 (#1888, "What
changed"; #2075, "Bit for bit": parity cases per KV format); its layout is this library's reading."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_attention_amd as qsa
import synth
from gpu_util import BLOCK, build_index, decode_layer, dev, rel_err_rows, to_device
from test_gpu_append import _host, _new_rows
from test_gpu_decode import _check_end_to_end, _partials_vs_oracle, dims_of, small_workload
from test_gpu_layer import run_layer

pytestmark = pytest.mark.gpu
TOL = 1e-5


@pytest.mark.parametrize("d,G,S", [(128, 6, 5), (128, 1, 3), (256, 3, 4), (256, 8, 7), (128, 8, 12), (192, 6, 4)])
def test_k8v4_chunk_partials(d, G, S):
    w = small_workload(2000 + d + G, n_kv=2, G=G, d=d, cap=1500, n_valid=1421, rows=3, topk=9, v_bits=4)
    dims = dims_of(w)
    pool = w.pools[0]
    nb = -(-pool.n_valid // BLOCK)
    s = oracle.block_scores(w.q, w.pos, oracle.block_index(pool), 2, pool.n_valid, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), w.topk)
    _partials_vs_oracle(w, to_device(pool), dims, S, ids.reshape(3, 2, -1), counts.reshape(3, 2))


@pytest.mark.parametrize("d,G,rows,topk,S", [(128, 6, 4, 7, 3), (256, 4, 3, 9, 5), (128, 2, 2, 20, 16),
                                             (192, 5, 3, 9, 4)])
def test_k8v4_layer_equals_separate_calls_and_oracle(d, G, rows, topk, S):
    w = small_workload(2100 + d + G, n_kv=2, G=G, d=d, cap=2100, n_valid=2010, rows=rows, topk=topk, v_bits=4)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    sep = decode_layer(w, p, dims, n_chunks=S)
    got = run_layer(w, [p], dims, S)
    assert np.array_equal(got["ids"], sep["ids"]) and np.array_equal(got["counts"], sep["counts"])
    assert rel_err_rows(got["out"], sep["out"]).max() <= TOL
    _check_end_to_end(w, got)


def test_k8v4_verify_window():
    """The verify window at full size (200,000-cell capacity, 16,384 valid cells) in K8V4."""
    w = synth.workload("verify_window", v_bits=4)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    _check_end_to_end(w, run_layer(w, [p], dims, 16))


def test_k8v4_dense_chunks():
    """Dense mode (fixed blocks per chunk, no selection) over a K8V4 pool: the merged output is dense attention."""
    w = synth.workload("drafter", v_bits=4, n_valid=4000, cap=4096, n_chunks=64, n_active=63)
    dims = dims_of(w)
    pool = w.pools[0]
    p = to_device(pool)
    part = qsa.Partials.empty_like_shape(1, dims.n_q_heads, w.n_chunks, dims.head_dim)
    qsa.qsa_attn_chunk(dev(w.q), dev(w.pos), [p], dims, part, w.n_chunks, w.sm_scale,
                       blocks_per_chunk=w.blocks_per_chunk)
    out = torch.empty(1, dims.n_q_heads, dims.head_dim, dtype=torch.float32, device="cuda")
    lse = torch.empty(1, dims.n_q_heads, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, w.n_chunks, out, lse)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attn(w.q, w.pos, pool, w.n_kv_heads)
    assert rel_err_rows(out.cpu().numpy(), ref).max() <= TOL
    assert np.abs(lse.cpu().numpy() - ref_lse).max() <= TOL * np.abs(ref_lse).max()


def test_k8v4_batch_window_two_pools():
    # seed 2400: every row's k-th and (k+1)-th FP64 block scores are apart by more than the fp32 error band
    w = synth.workload("batch_window", v_bits=4, seed=2400)
    dims = dims_of(w)
    pdevs = [build_index(to_device(pl), dims) for pl in w.pools]
    got = run_layer(w, pdevs, dims, 20, row_pool=dev(w.row_pool))
    for sidx in range(2):
        rows = slice(2 * sidx, 2 * sidx + 2)
        _check_end_to_end(w, {k: v[rows] for k, v in got.items()}, pool=w.pools[sidx], rows=rows)


def test_k8v4_mixed_formats_rejected():
    """Pools of different V formats in one call are refused before any launch."""
    a = synth.random_pool(2200, 1, 256, 256, 128)
    b = synth.random_pool(2201, 1, 256, 256, 128, v_bits=4)
    dims = qsa.Dims(2, 1, 128)
    pa, pb = to_device(a), to_device(b)
    part = qsa.Partials.empty_like_shape(2, 2, 2, 128)
    q = dev(synth.random_q(2202, 2, 2, 128))
    pos = dev(np.array([255, 255], np.int32))
    with pytest.raises(qsa.QSAError):
        qsa.qsa_attn_chunk(q, pos, [pa, pb], dims, part, 2, 1.0, row_pool=dev(np.array([0, 1], np.int32)),
                           blocks_per_chunk=2)


@pytest.mark.parametrize("d", [128, 192, 256])
def test_k8v4_append_matches_oracle_bitwise(d):
    n_kv, cap, n_old = 2, 700, 600
    pool = synth.random_pool(2300 + d, n_kv, cap, n_old, d, poison=False, v_bits=4)
    cells = np.array([600, 601, 640, 605, 699, 650], np.int32)
    n_new = 660
    kn, vn = _new_rows(2301 + d, len(cells), n_kv, d, zero_group=True)
    vn[1, 1, 64:128] = 0.0                                        # an all-zero V group
    dims = qsa.Dims(n_kv * 2, n_kv, d)
    p = to_device(pool)
    p.n_valid = n_new
    qsa.qsa_block_index(p, dims, 0, n_old, p.index)
    qsa.qsa_kv_append([p], dims, dev(kn), dev(vn), dev(cells))
    torch.cuda.synchronize()
    k, ks, v, vs, idx = _host(p)
    ref = oracle.kv_append(pool, kn, vn, cells, n_valid=n_new)
    assert v.shape[-1] == d // 2
    assert np.array_equal(k, ref.k) and np.array_equal(v, ref.v)
    assert np.array_equal(ks, ref.ks) and np.array_equal(vs, ref.vs)
    assert vs[1, 601, 1] == 0 and np.all(v[1, 601, 32:64] == 0)
    r = oracle.block_index(ref, n_blocks=-(-n_new // BLOCK))
    for b in (9, 10):
        assert rel_err_rows(idx[:, b], r[:, b]).max() <= TOL, b
