"""Parity of the append path (qsa_kv_append: int8 encode of new K/V cells, then the index rows of the blocks they
land in) against the oracle, through the C ABI. Codes and scales must match bit for bit (both sides decide them in
fp32); index rows within 1e-5 of the FP64 block means."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_attention_amd as qsa
import synth
from gpu_util import BLOCK, build_index, dev, rel_err_rows, to_device
from test_gpu_decode import _check_end_to_end, dims_of

pytestmark = pytest.mark.gpu
TOL = 1e-5


def _new_rows(seed, n_rows, n_kv, d, zero_group=False):
    rng = np.random.default_rng(seed)
    kn = (rng.standard_normal((n_rows, n_kv, d)) * rng.choice([0.01, 1.0, 50.0], (n_rows, n_kv, 1))).astype(np.float32)
    vn = (rng.standard_normal((n_rows, n_kv, d)) * 2.0).astype(np.float32)
    if zero_group:
        kn[0, 0, :64] = 0.0                                   # an all-zero group: scale 0, codes 0
    return kn, vn


def _host(p):
    return (p.k.cpu().numpy(), p.k_scale.cpu().numpy(), p.v.cpu().numpy(), p.v_scale.cpu().numpy(),
            p.index.cpu().numpy())


@pytest.mark.parametrize("d,many", [(64, False), (128, False), (192, False), (256, False), (64, True), (128, True)])
def test_append_matches_oracle_bitwise(d, many):
    """6 or 12 new rows (12 rows: six more cells in the same two blocks) against the oracle's encoder, bit for bit."""
    n_kv, cap, n_old = 2, 700, 600
    pool = synth.random_pool(1000 + d, n_kv, cap, n_old, d, poison=False)
    cells = np.array([600, 601, 640, 605, 699, 650], np.int32)   # rows share blocks; 699 >= n_valid: skipped
    if many:
        cells = np.concatenate([cells, np.array([602, 603, 641, 651, 659, 604], np.int32)])
    n_new = 660                                                    # n_valid after the append
    kn, vn = _new_rows(1001 + d, len(cells), n_kv, d, zero_group=True)
    dims = qsa.Dims(n_kv * 3, n_kv, d)
    p = to_device(pool)
    p.n_valid = n_new
    p.index = torch.full((n_kv, -(-cap // BLOCK), d), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_block_index(p, dims, 0, n_old, p.index)
    qsa.qsa_kv_append([p], dims, dev(kn), dev(vn), dev(cells))
    torch.cuda.synchronize()
    k, ks, v, vs, idx = _host(p)
    ref = oracle.kv_append(pool, kn, vn, cells, n_valid=n_new)
    # cells the oracle skipped or never touched keep the pool's bytes (the new cells beyond 600 start as zeros)
    assert np.array_equal(k, ref.k) and np.array_equal(v, ref.v)
    assert np.array_equal(ks, ref.ks) and np.array_equal(vs, ref.vs)
    assert np.all(ks[0, 600, 0] == 0) and np.all(k[0, 600, :64] == 0)
    # index rows of the blocks that received a cell: blocks 9 and 10 (cells 600..605, 640, 650)
    r = oracle.block_index(ref, n_blocks=-(-n_new // BLOCK))
    for b in (9, 10):
        assert rel_err_rows(idx[:, b], r[:, b]).max() <= TOL, b
    assert np.all(np.isnan(idx[:, 11:]))                        # no cell landed there: untouched


def test_append_two_pools_and_bad_rows():
    d, n_kv = 128, 2
    pools = [synth.random_pool(1100 + s, n_kv, 500, 400, d, poison=False) for s in range(2)]
    dims = qsa.Dims(6, n_kv, d)
    pdev = []
    for pl in pools:
        p = to_device(pl)
        p.n_valid = 420
        p.index = torch.zeros(n_kv, -(-500 // BLOCK), d, dtype=torch.float32, device="cuda")
        qsa.qsa_block_index(p, dims, 0, 400, p.index)
        pdev.append(p)
    cells = np.array([400, 401, 410, 419, 405], np.int32)
    row_pool = np.array([0, 1, 1, 0, 7], np.int32)                 # row 4 names no pool: skipped
    kn, vn = _new_rows(1102, 5, n_kv, d)
    qsa.qsa_kv_append(pdev, dims, dev(kn), dev(vn), dev(cells), row_pool=dev(row_pool))
    torch.cuda.synchronize()
    for s_ in range(2):
        rows = np.nonzero(row_pool == s_)[0]
        ref = oracle.kv_append(pools[s_], kn[rows], vn[rows], cells[rows], n_valid=420)
        k, ks, v, vs, idx = _host(pdev[s_])
        assert np.array_equal(k, ref.k) and np.array_equal(v, ref.v)
        assert np.array_equal(ks, ref.ks) and np.array_equal(vs, ref.vs)
        r = oracle.block_index(ref, n_blocks=7)
        assert rel_err_rows(idx[:, 6], r[:, 6]).max() <= TOL


def test_append_then_decode_layer():
    """Four new tokens appended to the verify-window pool (200,000-cell capacity), then the layer for queries at
    those positions: ids and outputs against the oracle on the appended pool."""
    w = synth.workload("verify_window", poison=False)
    pool = w.pools[0]
    dims = dims_of(w)
    n_old = pool.n_valid - 4                                   # the last 4 cells arrive by append
    p = to_device(pool)
    p.index = torch.zeros(w.n_kv_heads, -(-pool.capacity // BLOCK), w.head_dim, dtype=torch.float32,
                          device="cuda")
    p.n_valid = n_old
    qsa.qsa_block_index(p, dims, 0, n_old, p.index)
    cells = np.arange(n_old, n_old + 4, dtype=np.int32)
    kn, vn = _new_rows(1200, 4, w.n_kv_heads, w.head_dim)
    p.n_valid = pool.n_valid
    qsa.qsa_kv_append([p], dims, dev(kn), dev(vn), dev(cells))
    ref_pool = oracle.kv_append(pool, kn, vn, cells, n_valid=pool.n_valid)
    w2 = synth.Workload(w.name, w.n_q_heads, w.n_kv_heads, w.head_dim, [ref_pool], w.q, w.pos, w.row_pool, w.topk,
                        w.n_chunks, w.blocks_per_chunk, w.n_active, w.sm_scale)
    nb = -(-pool.n_valid // BLOCK)
    n_rows = w.q.shape[0]
    out = torch.empty(n_rows, dims.n_q_heads, dims.head_dim, dtype=torch.float32, device="cuda")
    lse = torch.empty(n_rows, dims.n_q_heads, dtype=torch.float32, device="cuda")
    scores = torch.empty(n_rows, dims.n_kv_heads, nb, dtype=torch.float32, device="cuda")
    ids = torch.empty(n_rows, dims.n_kv_heads, w.topk, dtype=torch.int32, device="cuda")
    counts = torch.empty(n_rows, dims.n_kv_heads, dtype=torch.int32, device="cuda")
    scratch = torch.empty(qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, nb, w.topk, 16), dtype=torch.uint8,
                          device="cuda")
    qsa.qsa_decode_layer(dev(w.q), dev(w.pos), [p], dims, nb, w.topk, 16, out, lse, sm_scale=w.sm_scale,
                         scores=scores, ids=ids, counts=counts, scratch=scratch)
    torch.cuda.synchronize()
    got = dict(scores=scores.cpu().numpy(), ids=ids.cpu().numpy(), counts=counts.cpu().numpy(),
               out=out.cpu().numpy(), lse=lse.cpu().numpy())
    _check_end_to_end(w2, got)
