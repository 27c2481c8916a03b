"""Parity of the decode-layer call (qsa_decode_layer: fused scores + top-k, then chunk attention, then the merge)
and of the fused selection (qsa_decode_select) against the separate calls and the FP64 oracle, through the C ABI."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_attention_amd as qsa
import synth
from gpu_util import BLOCK, build_index, decode_layer, dev, rel_err_rows, to_device
from test_gpu_decode import _check_end_to_end, dims_of, small_workload

pytestmark = pytest.mark.gpu
TOL = 1e-5


def run_layer(w, pdevs, dims, n_chunks, row_pool=None, nb=None, scratch=None, q=None, with_scores=True):
    n_rows = w.q.shape[0]
    nb = nb or -(-w.pools[0].n_valid // BLOCK)
    q = dev(w.q) if q is None else q
    out = torch.full((n_rows, dims.n_q_heads, dims.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    lse = torch.full((n_rows, dims.n_q_heads), float("nan"), dtype=torch.float32, device="cuda")
    scores = torch.empty(n_rows, dims.n_kv_heads, nb, dtype=torch.float32, device="cuda")
    ids = torch.empty(n_rows, dims.n_kv_heads, w.topk, dtype=torch.int32, device="cuda")
    counts = torch.empty(n_rows, dims.n_kv_heads, dtype=torch.int32, device="cuda")
    if scratch is None:
        scratch = torch.empty(qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, nb, w.topk, n_chunks), dtype=torch.uint8,
                              device="cuda")
    qsa.qsa_decode_layer(q, dev(w.pos), pdevs, dims, nb, w.topk, n_chunks, out, lse, sm_scale=w.sm_scale,
                         row_pool=row_pool, scores=scores if with_scores else None, ids=ids, counts=counts,
                         scratch=scratch)
    torch.cuda.synchronize()
    return dict(scores=scores.cpu().numpy() if with_scores else None, ids=ids.cpu().numpy(), counts=counts.cpu().numpy(),
                out=out.cpu().numpy(), lse=lse.cpu().numpy())


@pytest.mark.parametrize("d,G,rows,topk,S", [(128, 6, 4, 7, 3), (64, 1, 2, 5, 8), (256, 8, 3, 9, 2),
                                             (128, 5, 5, 12, 5), (128, 3, 2, 4, 9), (192, 6, 3, 8, 3)])
def test_layer_equals_separate_calls_and_oracle(d, G, rows, topk, S):
    w = small_workload(500 + d + G, n_kv=2, G=G, d=d, cap=2100, n_valid=2010, rows=rows, topk=topk)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    sep = decode_layer(w, p, dims, n_chunks=S)
    got = run_layer(w, [p], dims, S)
    # the select launch does the separate calls' arithmetic: the same score bits, ids and counts
    assert np.array_equal(got["scores"], sep["scores"])
    assert np.array_equal(got["ids"], sep["ids"]) and np.array_equal(got["counts"], sep["counts"])
    assert rel_err_rows(got["out"], sep["out"]).max() <= TOL
    _check_end_to_end(w, got)


@pytest.mark.parametrize("S", [16, 8, 33])
def test_layer_verify_window(S):
    """The verify window at full size (200,000-cell capacity), with more chunks than blocks when S = 33."""
    w = synth.workload("verify_window")
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    got = run_layer(w, [p], dims, S)
    _check_end_to_end(w, got)


@pytest.mark.parametrize("S,v_bits", [(16, 8), (4, 8), (16, 4)])
def test_layer_head_dim_192_verify_window_shape(S, v_bits):
    """head_dim 192 (the lane layouts of 256 with the slices past dim 191 empty) on the verify window's shape: 4 rows
    at the last positions, 24/4 heads, 16,384 valid cells, top-32; with 4 chunks every wave takes several pieces."""
    # (seed 701: every row's k-th score margin clears the fp32 error band, for both V formats)
    w = small_workload(701, n_kv=4, G=6, d=192, cap=20_000, n_valid=16_384, rows=4, topk=32, v_bits=v_bits)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    got = run_layer(w, [p], dims, S)
    _check_end_to_end(w, got)


def test_layer_repeated_calls_reuse_scratch():
    """Back-to-back calls on one scratch buffer, with different q, all match."""
    w = small_workload(611, n_kv=2, G=6, rows=3, topk=8)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    scratch = torch.empty(qsa.qsa_decode_layer_scratch_bytes(3, dims, -(-w.pools[0].n_valid // BLOCK), w.topk, 4), dtype=torch.uint8, device="cuda")
    for rep in range(3):
        w.q = synth.random_q(700 + rep, 3, dims.n_q_heads, dims.head_dim)
        got = run_layer(w, [p], dims, 4, scratch=scratch)
        _check_end_to_end(w, got)


@pytest.mark.parametrize("S", [20, 32])
def test_layer_batch_window_two_pools(S):
    """Both slots' rows in one call through row_pool (32 chunks is the split the benchmark times); each slot checked
    against the oracle on its own pool."""
    w = synth.workload("batch_window")
    dims = dims_of(w)
    pdevs = [build_index(to_device(pl), dims) for pl in w.pools]
    got = run_layer(w, pdevs, dims, S, row_pool=dev(w.row_pool))
    for sidx in range(2):
        rows = slice(2 * sidx, 2 * sidx + 2)
        sub = {k: v[rows] for k, v in got.items()}
        _check_end_to_end(w, sub, pool=w.pools[sidx], rows=rows)


def test_wide_rows_split_selection_matches_fused():
    """Rows of 1,024 blocks over two pools, one row with an out-of-range pool index: the selection through a score
    buffer (score rows in one launch, then the top-k) picks the ids and counts of the fused one-launch selection, and
    the layer gives the same bits with or without a caller's score buffer."""
    w = synth.workload("batch_window")
    dims = dims_of(w)
    pdevs = [build_index(to_device(pl), dims) for pl in w.pools]
    rp = w.row_pool.copy()
    rp[1] = 7
    rpd = dev(rp)
    nb = -(-w.pools[0].n_valid // BLOCK)
    assert nb > 256
    q, pos = dev(w.q), dev(w.pos)
    n_rows = w.q.shape[0]
    res = []
    for with_scores in (False, True):
        s = torch.full((n_rows, dims.n_kv_heads, nb), float("nan"), dtype=torch.float32, device="cuda")
        i = torch.empty(n_rows, dims.n_kv_heads, w.topk, dtype=torch.int32, device="cuda")
        c = torch.empty(n_rows, dims.n_kv_heads, dtype=torch.int32, device="cuda")
        qsa.qsa_decode_select(q, pos, pdevs, dims, nb, w.topk, i, c, row_pool=rpd, scores=s if with_scores else None)
        torch.cuda.synchronize()
        res.append((i.cpu().numpy(), c.cpu().numpy(), s.cpu().numpy()))
    assert np.array_equal(res[0][0], res[1][0]) and np.array_equal(res[0][1], res[1][1])
    assert np.all(res[1][1][1] == 0) and np.all(np.isneginf(res[1][2][1]))
    # the split path's ids: the oracle's top-k of its own fp32 score rows
    ids2, cnt2 = oracle.topk(res[1][2].astype(np.float64).reshape(-1, nb), w.topk)
    assert np.array_equal(res[1][0].reshape(-1, w.topk), ids2) and np.array_equal(res[1][1].reshape(-1), cnt2)
    with_buf = run_layer(w, pdevs, dims, 32, row_pool=rpd)
    without = run_layer(w, pdevs, dims, 32, row_pool=rpd, with_scores=False)
    for key in ("ids", "counts", "out", "lse"):
        assert np.array_equal(with_buf[key], without[key]), key
    assert np.array_equal(with_buf["ids"], res[1][0])


@pytest.mark.parametrize("d,G,topk,n_valid,extra", [(128, 6, 200, 15_000, 0), (128, 2, 100, 15_000, 0),
                                                    (64, 4, 256, 60_000, 0), (128, 6, 40, 15_000, 900)])
def test_layer_large_k_and_width_limits(d, G, topk, n_valid, extra):
    """Selections past 64 ids (read from LDS by the chunk workgroups), k at the fused limit of 256, and rows just past
    the fused width limit (1,135 columns: the selection launch, then the chunks read the ids): the same ids, counts
    and output as the separate calls."""
    w = small_workload(900 + topk + G, n_kv=2, G=G, d=d, cap=n_valid + 64 * extra + 64, n_valid=n_valid, rows=3,
                       topk=topk)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    nb = -(-n_valid // BLOCK) + extra
    sep = decode_layer(w, p, dims, n_chunks=5, nb=nb)
    got = run_layer(w, [p], dims, 5, nb=nb)
    assert np.array_equal(got["scores"], sep["scores"])
    assert np.array_equal(got["ids"], sep["ids"]) and np.array_equal(got["counts"], sep["counts"])
    assert rel_err_rows(got["out"], sep["out"]).max() <= TOL


def test_layer_verify_window_four_slots_four_chunks():
    """Four verify-window slots (one 200,000-cell pool each) in one call with 4 chunks per row, the launch shape of
    the benchmark's scale measurement: every wave of the chunk kernel takes several pieces."""
    w = synth.workload("verify_window", slots=4)
    dims = dims_of(w)
    pdevs = [build_index(to_device(pl), dims) for pl in w.pools]
    got = run_layer(w, pdevs, dims, 4, row_pool=dev(w.row_pool))
    for sidx in range(4):
        rows = slice(4 * sidx, 4 * sidx + 4)
        sub = {k: v[rows] for k, v in got.items()}
        _check_end_to_end(w, sub, pool=w.pools[sidx], rows=rows)


def test_layer_bad_row_pool_gives_empty_rows():
    """A row whose device-side pool index is out of range selects nothing: zero output, lse -inf."""
    w = small_workload(623, n_kv=2, G=3, rows=3, topk=6)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    got = run_layer(w, [p], dims, 4, row_pool=dev(np.array([0, 5, 0], np.int32)))
    assert np.all(got["counts"][1] == 0) and np.all(got["ids"][1] == -1)
    assert np.all(got["out"][1] == 0) and np.all(np.isneginf(got["lse"][1]))
    sub = {k: v[[0, 2]] for k, v in got.items()}
    w2 = synth.Workload("rows02", w.n_q_heads, w.n_kv_heads, w.head_dim, w.pools, w.q[[0, 2]], w.pos[[0, 2]],
                        w.row_pool[[0, 2]], w.topk, w.n_chunks, w.blocks_per_chunk, w.n_active, w.sm_scale)
    _check_end_to_end(w2, sub)


def test_layer_first_position_sees_one_block():
    """A row at position 0 sees one cell: one eligible block, the rest of its ids -1."""
    w = small_workload(631, n_kv=2, G=2, rows=2, topk=5)
    w.pos = np.array([0, 700], np.int32)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    got = run_layer(w, [p], dims, 3)
    assert np.all(got["counts"][0] == 1) and np.all(got["ids"][0][:, 1:] == -1)
    _check_end_to_end(w, got)


@pytest.mark.parametrize("d,G,width_extra", [(128, 6, 0), (64, 2, 1), (256, 4, 0), (192, 3, 1)])
def test_select_equals_separate_calls(d, G, width_extra):
    """qsa_decode_select gives the bits of qsa_block_scores + qsa_topk, with or without a score output, and on
    score rows wider than the valid blocks (extra columns are -inf)."""
    w = small_workload(640 + d + G, n_kv=2, G=G, d=d, cap=2100, n_valid=2010, rows=3, topk=9)
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    nb = -(-w.pools[0].n_valid // BLOCK) + width_extra
    q, pos = dev(w.q), dev(w.pos)
    s_sep = torch.empty(3, 2, nb, dtype=torch.float32, device="cuda")
    qsa.qsa_block_scores(q, pos, p, dims, nb, s_sep)
    i_sep = torch.empty(3, 2, w.topk, dtype=torch.int32, device="cuda")
    c_sep = torch.empty(3, 2, dtype=torch.int32, device="cuda")
    qsa.qsa_topk(s_sep, w.topk, i_sep, c_sep)
    for with_scores in (True, False):
        s = torch.full((3, 2, nb), float("nan"), dtype=torch.float32, device="cuda") if with_scores else None
        i = torch.empty(3, 2, w.topk, dtype=torch.int32, device="cuda")
        c = torch.empty(3, 2, dtype=torch.int32, device="cuda")
        qsa.qsa_decode_select(q, pos, [p], dims, nb, w.topk, i, c, scores=s)
        torch.cuda.synchronize()
        if with_scores:
            assert np.array_equal(s.cpu().numpy(), s_sep.cpu().numpy())
        assert np.array_equal(i.cpu().numpy(), i_sep.cpu().numpy())
        assert np.array_equal(c.cpu().numpy(), c_sep.cpu().numpy())


def test_select_wide_rows():
    """Score rows of 5,000 blocks (more than 16 per thread): the same ids as the separate calls."""
    pool = synth.random_pool(651, 1, 320_000, 320_000, 64)
    w = synth.Workload("wide", 2, 1, 64, [pool], synth.random_q(652, 2, 2, 64), np.array([319_999, 250_000], np.int32),
                       np.zeros(2, np.int32), 40, 4, 1, 0, 1.0)
    dims = dims_of(w)
    p = build_index(to_device(pool), dims)
    nb = 5000
    q, pos = dev(w.q), dev(w.pos)
    s_sep = torch.empty(2, 1, nb, dtype=torch.float32, device="cuda")
    qsa.qsa_block_scores(q, pos, p, dims, nb, s_sep)
    i_sep = torch.empty(2, 1, 40, dtype=torch.int32, device="cuda")
    c_sep = torch.empty(2, 1, dtype=torch.int32, device="cuda")
    qsa.qsa_topk(s_sep, 40, i_sep, c_sep)
    i = torch.empty_like(i_sep)
    c = torch.empty_like(c_sep)
    qsa.qsa_decode_select(q, pos, [p], dims, nb, 40, i, c)
    torch.cuda.synchronize()
    assert np.array_equal(i.cpu().numpy(), i_sep.cpu().numpy()) and np.array_equal(c.cpu().numpy(), c_sep.cpu().numpy())


def test_capacity_wide_selection():
    """Score rows over the whole 200,000-cell capacity (3,125 blocks, -inf past n_valid) select what rows over the
    valid blocks select, and the layer output is the same."""
    w = synth.workload("verify_window")
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    nb_valid = -(-w.pools[0].n_valid // BLOCK)
    nb_cap = -(-w.pools[0].capacity // BLOCK)
    narrow = run_layer(w, [p], dims, 16, nb=nb_valid)
    wide = run_layer(w, [p], dims, 16, nb=nb_cap)
    assert wide["scores"].shape[-1] == 3125
    assert np.array_equal(wide["scores"][..., :nb_valid], narrow["scores"])
    assert np.all(np.isneginf(wide["scores"][..., nb_valid:]))
    assert np.array_equal(wide["ids"], narrow["ids"]) and np.array_equal(wide["counts"], narrow["counts"])
    assert np.array_equal(wide["out"], narrow["out"])
    _check_end_to_end(w, narrow)


@pytest.mark.parametrize("n_valid,topk", [(25_000, 20), (60_000, 64), (16_384, 256)])
def test_select_one_wave_topk_widths(n_valid, topk):
    """Score rows of 391 and 938 blocks (the one-wave top-k with 8 and 16 keys per lane), a row whose k equals its
    eligible count and a row of equal scores: the fused selection picks exactly what the separate score and top-k
    calls pick, and what the oracle's top-k of those scores picks."""
    pool = synth.random_pool(660 + topk, 2, n_valid + 64, n_valid, 128, poison=False)
    q = synth.random_q(661 + topk, 3, 12, 128)
    q[2, :6] = 0.0                      # row 2, KV head 0: every score is zero, a row of ties
    pos = np.array([n_valid - 1, n_valid // 2, 300], np.int32)
    dims = qsa.Dims(12, 2, 128)
    p = build_index(to_device(pool), dims)
    nb = -(-n_valid // BLOCK)
    qd, posd = dev(q), dev(pos)
    s_sep = torch.empty(3, 2, nb, dtype=torch.float32, device="cuda")
    qsa.qsa_block_scores(qd, posd, p, dims, nb, s_sep)
    i_sep = torch.empty(3, 2, topk, dtype=torch.int32, device="cuda")
    c_sep = torch.empty(3, 2, dtype=torch.int32, device="cuda")
    qsa.qsa_topk(s_sep, topk, i_sep, c_sep)
    i = torch.empty_like(i_sep)
    c = torch.empty_like(c_sep)
    qsa.qsa_decode_select(qd, posd, [p], dims, nb, topk, i, c)
    torch.cuda.synchronize()
    assert np.array_equal(i.cpu().numpy(), i_sep.cpu().numpy()) and np.array_equal(c.cpu().numpy(), c_sep.cpu().numpy())
    ref, cnt = oracle.topk(s_sep.cpu().numpy().astype(np.float64).reshape(-1, nb), topk)
    assert np.array_equal(i.cpu().numpy().reshape(-1, topk), ref) and np.array_equal(c.cpu().numpy().reshape(-1), cnt)
