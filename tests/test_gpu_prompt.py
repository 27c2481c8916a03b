"""Parity of the int8-MFMA prompt-chunk attention against the FP64 oracle (dense causal attention), through the
C ABI, for int8 and K8V4 pools. Bar: max relative error 1e-5 per (query, head) row. Pools carry poison past
n_valid."""
import numpy as np
import pytest
import torch

import oracle
import sparse_top_attention_amd as qsa
import synth
from gpu_util import dev, rel_err_rows, to_device

pytestmark = pytest.mark.gpu
TOL = 1e-5


def run_prompt(q, pos0, p_dev, dims, sm_scale=1.0):
    n_q = q.shape[0]
    nbytes = qsa.qsa_prompt_scratch_bytes(n_q, pos0, dims)
    scratch = torch.empty(max(nbytes, 1), dtype=torch.uint8, device="cuda")
    out = torch.full((n_q, dims.n_q_heads, dims.head_dim), float("nan"), dtype=torch.float32, device="cuda")
    qsa.qsa_prompt_attn(dev(q), pos0, p_dev, dims, out, sm_scale=sm_scale, scratch=scratch)
    torch.cuda.synchronize()
    return out.cpu().numpy()


@pytest.mark.parametrize("v_bits", [8, 4], ids=["int8", "k8v4"])
@pytest.mark.parametrize("n_kv,G,n_q,pos0,n_valid,cap", [
    (4, 6, 70, 300, 400, 420),       # 24/4 heads, ragged tile tails, several workgroups
    (2, 6, 11, 0, 700, 700),         # the first query sees one cell
    (4, 6, 40, 380, 400, 450),       # queries past n_valid see every valid cell
    (1, 1, 130, 500, 640, 640),
    (2, 2, 33, 64, 97, 128),
    (2, 8, 50, 1000, 1049, 1100),
])
def test_prompt_small(n_kv, G, n_q, pos0, n_valid, cap, v_bits):
    """head_dim 128 on the matrix-core kernel; a K8V4 pool's 4-bit V codes are widened to int8 in LDS."""
    pool = synth.random_pool(300 + n_q + v_bits, n_kv, cap, n_valid, 128, v_bits=v_bits)
    q = synth.random_q(301 + n_q, n_q, n_kv * G, 128)
    dims = qsa.Dims(n_kv * G, n_kv, 128)
    got = run_prompt(q, pos0, to_device(pool), dims)
    pos = (pos0 + np.arange(n_q)).astype(np.int32)
    ref, _ = oracle.attn(q, pos, pool, n_kv)
    assert np.all(np.isfinite(got))
    assert rel_err_rows(got, ref).max() <= TOL


@pytest.mark.parametrize("d,v_bits,n_kv,G,n_q,pos0,n_valid,cap", [
    (64, 8, 2, 6, 130, 300, 400, 420),        # three 64-query batches, queries past n_valid
    (256, 8, 2, 3, 70, 1000, 1049, 1100),     # head_dim 256, a ragged last block
    (256, 4, 1, 8, 40, 0, 2100, 2100),        # K8V4 at 256, the first query sees one cell
    (192, 8, 2, 6, 90, 700, 760, 800),        # head_dim 192 (lanes of the 256 layout), two batches
    (192, 4, 1, 3, 20, 1200, 1290, 1300),     # K8V4 at 192
])
def test_prompt_other_shapes_match_oracle(d, v_bits, n_kv, G, n_q, pos0, n_valid, cap):
    """Head dims without the int8 matrix-core kernel (64, 192 and 256) take the dense chunk path: the same causal
    attention, checked against the FP64 oracle on every row."""
    pool = synth.random_pool(360 + d + v_bits, n_kv, cap, n_valid, d, v_bits=v_bits)
    q = synth.random_q(361 + d, n_q, n_kv * G, d)
    dims = qsa.Dims(n_kv * G, n_kv, d)
    got = run_prompt(q, pos0, to_device(pool), dims, sm_scale=0.9)
    pos = (pos0 + np.arange(n_q)).astype(np.int32)
    ref, _ = oracle.attn(q, pos, pool, n_kv, sm_scale=0.9)
    assert np.all(np.isfinite(got))
    assert rel_err_rows(got, ref).max() <= TOL


@pytest.mark.parametrize("v_bits", [8, 4], ids=["int8", "k8v4"])
def test_prompt_edge_cases(v_bits):
    """A pool with no valid cell (every row sees nothing: zeros), a single query, and a negative scale."""
    dims = qsa.Dims(12, 2, 128)
    empty = synth.random_pool(351, 2, 256, 0, 128, v_bits=v_bits)
    q = synth.random_q(352, 40, 12, 128)
    got = run_prompt(q, 100, to_device(empty), dims)
    assert np.all(got == 0.0)
    pool = synth.random_pool(353, 2, 900, 700, 128, v_bits=v_bits)
    p = to_device(pool)
    for n_q, pos0, scale in [(1, 0, 1.0), (1, 699, 1.0), (1, 5000, 0.8), (70, 600, -0.6),
                             (3, 2**31 - 3, 1.0)]:   # the last query at position INT32_MAX sees every valid cell
        q = synth.random_q(354 + n_q + pos0, n_q, 12, 128)
        got = run_prompt(q, pos0, p, dims, sm_scale=scale)
        pos = (pos0 + np.arange(n_q)).astype(np.int32)
        ref, _ = oracle.attn(q, pos, pool, 2, sm_scale=scale)
        assert rel_err_rows(got, ref).max() <= TOL, (n_q, pos0, scale)


@pytest.mark.parametrize("v_bits", [8, 4], ids=["int8", "k8v4"])
def test_prompt_rising_logits_fold_many_times(v_bits):
    """Key scales ramping 12x along the context make each row's max keep rising, so the int32 sums are folded into
    the stored output again and again (5 to 10 times per row: each time the max passes the reference), with
    rescales between folds. The logits stay within about +-80 (log2 units), where fp32 logits still meet the bar."""
    n_kv, G, n_q, pos0, n_valid = 2, 6, 64, 1500, 1564
    pool = synth.random_pool(361 + v_bits, n_kv, n_valid, n_valid, 128, v_bits=v_bits)
    ramp = np.linspace(1.0, 12.0, n_valid, dtype=np.float32)[None, :, None]
    pool.ks[:] = pool.ks * ramp
    q = synth.random_q(362, n_q, n_kv * G, 128)
    dims = qsa.Dims(n_kv * G, n_kv, 128)
    got = run_prompt(q, pos0, to_device(pool), dims)
    pos = (pos0 + np.arange(n_q)).astype(np.int32)
    ref, _ = oracle.attn(q, pos, pool, n_kv)
    assert np.all(np.isfinite(got))
    assert rel_err_rows(got, ref).max() <= TOL


def test_prompt_sm_scale_and_zero_query():
    pool = synth.random_pool(311, 2, 300, 260, 128)
    q = synth.random_q(312, 20, 12, 128)
    q[3] = 0.0                                            # all-zero rows: uniform weights
    dims = qsa.Dims(12, 2, 128)
    got = run_prompt(q, 230, to_device(pool), dims, sm_scale=0.37)
    pos = (230 + np.arange(20)).astype(np.int32)
    ref, _ = oracle.attn(q, pos, pool, 2, sm_scale=0.37)
    assert rel_err_rows(got, ref).max() <= TOL


def test_prompt_single_chunk_path():
    """8 KV heads x 4,096 queries: enough workgroups that the kernel writes the output without split chunks."""
    n_kv, G, n_q, pos0, n_valid = 8, 1, 4096, 100, 4200
    dims = qsa.Dims(n_kv * G, n_kv, 128)
    pool = synth.random_pool(321, n_kv, n_valid, n_valid, 128)
    q = synth.random_q(322, n_q, n_kv * G, 128)
    got = run_prompt(q, pos0, to_device(pool), dims)
    assert np.all(np.isfinite(got))
    pos = (pos0 + np.arange(n_q)).astype(np.int32)
    rng = np.random.default_rng(5)
    for i in list(rng.integers(0, n_q, 10)) + [0, n_q - 1]:
        for h in (0, 7):
            ref, _ = oracle.attn_one(q, pos, int(i), h, pool, n_kv)
            assert rel_err_rows(got[i, h][None], ref[None]).max() <= TOL, (i, h)


@pytest.mark.parametrize("v_bits", [8, 4], ids=["int8", "k8v4"])
def test_prompt_forced_fold_past_1024_tiles(v_bits):
    """One cell chunk longer than 1,024 tiles of 64 cells: the PV int32 sums are folded into fp32 every 1,024
    tiles whether or not the row max moved (8 KV heads x 4,096 queries fill the chip without splitting the cells,
    and pos0 = 66,000 gives every workgroup at least 1,032 tiles). Checked on sampled rows."""
    n_kv, G, n_q, pos0 = 8, 1, 4096, 66000
    n_valid = pos0 + n_q
    dims = qsa.Dims(n_kv * G, n_kv, 128)
    pool = synth.random_pool(341, n_kv, n_valid + 40, n_valid, 128, v_bits=v_bits)
    q = synth.random_q(342, n_q, n_kv * G, 128)
    got = run_prompt(q, pos0, to_device(pool), dims)
    assert np.all(np.isfinite(got))
    pos = (pos0 + np.arange(n_q)).astype(np.int32)
    rng = np.random.default_rng(9)
    picks = [(0, 0), (63, 3), (64, 4), (4095, 7), (4032, 1)]
    picks += [(int(i), int(h)) for i, h in zip(rng.integers(0, n_q, 11), rng.integers(0, n_kv, 11))]
    for i, h in picks:
        ref, _ = oracle.attn_one(q, pos, i, h, pool, n_kv)
        assert rel_err_rows(got[i, h][None], ref[None]).max() <= TOL, (i, h)


@pytest.mark.parametrize("v_bits", [8, 4], ids=["int8", "k8v4"])
def test_prompt_chunk_full_size_sampled(v_bits):
    """The 2,048-query prompt chunk at the end of a 32,768-cell context, checked on sampled rows."""
    w = synth.workload("prompt_chunk", v_bits=v_bits)
    pool = w.pools[0]
    dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
    got = run_prompt(w.q, w.pos0, to_device(pool), dims)
    assert np.all(np.isfinite(got))
    rng = np.random.default_rng(7)
    picks = [(0, 0), (1, 23), (63, 5), (64, 6), (1023, 11), (2047, 17), (2047, 0)]
    picks += [(int(i), int(h)) for i, h in zip(rng.integers(0, 2048, 33), rng.integers(0, 24, 33))]
    errs = []
    for i, h in picks:
        ref, _ = oracle.attn_one(w.q, w.pos, i, h, pool, w.n_kv_heads)
        errs.append(rel_err_rows(got[i, h][None], ref[None]).max())
        assert errs[-1] <= TOL, (i, h)
    print(f"prompt_chunk (v_bits {v_bits}) sampled rows: max rel err {max(errs):.3e} over {len(picks)} rows")


def test_prompt_last_row_equals_dense_decode():
    """The prompt's last query is an ordinary dense decode over the whole context: compare it with the chunk
    attention and merge run densely over the same pool."""
    w = synth.workload("prompt_chunk", n_valid=4096, cap=4096, rows=256)
    pool = w.pools[0]
    dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
    p = to_device(pool)
    got = run_prompt(w.q, w.pos0, p, dims)
    q_last = dev(w.q[-1:])
    pos_last = dev(w.pos[-1:])
    part = qsa.Partials.empty_like_shape(1, w.n_q_heads, 64, 128)
    qsa.qsa_attn_chunk(q_last, pos_last, [p], dims, part, 64, 1.0, blocks_per_chunk=1)
    out = torch.empty(1, w.n_q_heads, 128, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, 64, out)
    torch.cuda.synchronize()
    assert rel_err_rows(got[-1:], out.cpu().numpy()).max() <= 2 * TOL


def test_prompt_scratch_too_small_is_rejected():
    pool = synth.random_pool(331, 2, 300, 260, 128)
    dims = qsa.Dims(12, 2, 128)
    n = qsa.qsa_prompt_scratch_bytes(20, 230, dims)
    scratch = torch.empty(n - 1, dtype=torch.uint8, device="cuda")
    out = torch.empty(20, 12, 128, dtype=torch.float32, device="cuda")
    with pytest.raises(qsa.QSAError) as e:
        qsa.qsa_prompt_attn(dev(synth.random_q(1, 20, 12, 128)), 230, to_device(pool), dims, out, scratch=scratch)
    assert e.value.status == -4
