"""Pins for the FP64 oracle (CPU only): each check ties the oracle to something other than itself.

* brute force: textbook softmax(q K^T) V on tiny inputs, with every eligible block selected;
* split invariance: chunk partials for several split counts, merged, equal the unsplit attention;
* top-k: equal to Python's stable sort on tie-heavy rows, all-equal rows, all -inf rows, k >= width;
* closed forms: constant V, all-zero K, one dominant cell, q = 0;
* score identity: (sum of a group's q heads) . (block mean key) = the mean of the per-cell, per-head logits;
* merge algebra: empty or out-of-range chunks change nothing, bit for bit;
* the 24-bit split: exact for every integer in range, error of the scaling step within 2^-17;
* the int8 encoder (append path): nearest code by brute force over all 255 codes, exact recovery of power-of-two
  grids, the reconstruction bound, and appends that touch only their cells.
"""
import math

import numpy as np
import pytest

import brute
import oracle
import synth

B = oracle.BLOCK


def small_case(seed, n_kv=2, G=3, d=64, cap=300, n_valid=290, rows=3, poison=True):
    pool = synth.random_pool(seed, n_kv, cap, n_valid, d, poison=poison)
    q = synth.random_q(seed + 1, rows, n_kv * G, d)
    pos = np.array([n_valid - rows + r for r in range(rows)], np.int32)
    return pool, q, pos


# ---------------------------------------------------------------------------------------------------------------
# brute force
# ---------------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("d,n_valid,positions", [
    (64, 290, [289, 288, 200]),      # ragged last block, a query inside a block
    (128, 256, [255, 63, 64]),       # exact blocks, queries at a block's last and a block's first cell
    (64, 70, [0, 5, 69]),            # query at cell 0 sees one cell
    (192, 150, [149, 64, 100]),      # three scale groups per cell
])
def test_dense_equals_textbook(d, n_valid, positions):
    pool, q, _ = small_case(11, d=d, cap=n_valid + 17, n_valid=n_valid, rows=len(positions))
    pos = np.array(positions, np.int32)
    out, lse = oracle.attn(q, pos, pool, n_kv=2)
    ref = brute.textbook_attention(q, pos, pool)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    assert np.all(np.isfinite(lse))


def test_full_selection_equals_textbook():
    """k >= the number of blocks: the top-k keeps every eligible block, so selection attention is dense attention."""
    pool, q, pos = small_case(21, d=128, cap=520, n_valid=500, rows=3)
    nb = -(-pool.n_valid // B)
    r = oracle.block_index(pool)
    s = oracle.block_scores(q, pos, r, 2, pool.n_valid, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), k=nb + 3)
    ids = ids.reshape(3, 2, nb + 3)
    counts = counts.reshape(3, 2)
    out, _ = oracle.attn(q, pos, pool, 2, ids=ids, counts=counts)
    ref = brute.textbook_attention(q, pos, pool)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_sparse_equals_textbook_on_selected_blocks():
    pool, q, pos = small_case(31, d=64, cap=600, n_valid=600, rows=2)
    nb = -(-pool.n_valid // B)
    r = oracle.block_index(pool)
    s = oracle.block_scores(q, pos, r, 2, pool.n_valid, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), k=3)
    ids = ids.reshape(2, 2, 3)
    counts = counts.reshape(2, 2)
    sel = [[set(int(b) for b in ids[i, g] if b >= 0) for g in range(2)] for i in range(2)]
    out, _ = oracle.attn(q, pos, pool, 2, ids=ids, counts=counts)
    ref = brute.textbook_attention(q, pos, pool, selected_blocks=sel)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_dense_matches_matrix_form_medium():
    pool, q, pos = small_case(41, n_kv=2, G=2, d=128, cap=3000, n_valid=2900, rows=5)
    out, _ = oracle.attn(q, pos, pool, 2)
    ref = brute.matrix_attention(q, pos, pool)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


def test_attn_one_matches_attn():
    pool, q, pos = small_case(43)
    out, lse = oracle.attn(q, pos, pool, 2)
    for i, h in [(0, 0), (2, 5), (1, 3)]:
        o1, l1 = oracle.attn_one(q, pos, i, h, pool, 2)
        assert np.array_equal(o1, out[i, h]) and l1 == lse[i, h]


def test_lse_is_log_of_partition_function():
    pool, q, pos = small_case(47, d=64, n_valid=130, cap=140, rows=1)
    _, lse = oracle.attn(q, pos, pool, 2)
    K = brute.repeat_kv(brute.dequant(pool.k[:, :130], pool.ks[:, :130]), 6)
    for h in range(6):
        t = [float(np.dot(q[0, h].astype(np.float64), K[h, c])) for c in range(pos[0] + 1)]
        mx = max(t)
        assert abs(lse[0, h] - (mx + math.log(math.fsum(math.exp(x - mx) for x in t)))) < 1e-12


# ---------------------------------------------------------------------------------------------------------------
# split invariance and merge algebra
# ---------------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("S", [1, 2, 3, 5, 20])
def test_split_invariance_sparse(S):
    pool, q, pos = small_case(51, d=64, cap=1300, n_valid=1290, rows=3)
    nb = -(-pool.n_valid // B)
    r = oracle.block_index(pool)
    s = oracle.block_scores(q, pos, r, 2, pool.n_valid, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), k=7)
    ids, counts = ids.reshape(3, 2, 7), counts.reshape(3, 2)
    ref, ref_lse = oracle.attn(q, pos, pool, 2, ids=ids, counts=counts)
    m, l, o, e = oracle.chunk_partials(q, pos, pool, 2, S, ids=ids, counts=counts)
    out, lse = oracle.merge(m, l, o, e)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=0, atol=1e-12)
    # chunks past the row's selected blocks are empty, the others hold at least one cell here
    for i in range(3):
        for h in range(6):
            n_sel = counts[i, h // 3]
            assert e[i, h, :n_sel].sum() == 0 or S > n_sel
            assert np.all(e[i, h, min(S, n_sel):] == 1)


def test_split_invariance_one_block_per_chunk():
    pool, q, pos = small_case(53, d=128, cap=700, n_valid=650, rows=2)
    nb = -(-pool.n_valid // B)
    ids, counts = oracle.full_selection(pos, 2, pool.n_valid, nb)
    ref, _ = oracle.attn(q, pos, pool, 2, ids=ids, counts=counts)
    m, l, o, e = oracle.chunk_partials(q, pos, pool, 2, nb, ids=ids, counts=counts)
    out, _ = oracle.merge(m, l, o, e)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)


@pytest.mark.parametrize("bpc", [1, 2, 3])
def test_split_invariance_dense(bpc):
    pool, q, pos = small_case(57, d=64, cap=1000, n_valid=700, rows=2)
    S = -(-1000 // (B * bpc))
    n_active = np.full(2, -(-700 // (B * bpc)), np.int32)
    ref, _ = oracle.attn(q, pos, pool, 2)
    m, l, o, e = oracle.chunk_partials(q, pos, pool, 2, S, bpc=bpc)
    out, _ = oracle.merge(m, l, o, e, n_active=n_active)
    np.testing.assert_allclose(out, ref, rtol=0, atol=1e-12)
    assert np.all(e[:, :, n_active[0]:] == 1)


def test_merge_skips_marked_and_inactive_chunks_bitwise():
    pool, q, pos = small_case(61, d=64, cap=900, n_valid=900, rows=2)
    m, l, o, e = oracle.chunk_partials(q, pos, pool, 2, 5, bpc=3)
    out, lse = oracle.merge(m, l, o, e)
    # interleave garbage chunks that are marked empty, and append unmarked garbage past n_active
    S2 = 12
    m2 = np.full(m.shape[:2] + (S2,), 1000.0)    # a max that would swamp every real chunk if it were read
    l2 = np.full_like(m2, np.nan)
    o2 = np.full(o.shape[:2] + (S2, o.shape[3]), np.nan)
    e2 = np.ones(m2.shape, np.uint8)
    slots = [0, 2, 3, 6, 8]
    for j, sj in enumerate(slots):
        m2[..., sj], l2[..., sj], o2[..., sj, :], e2[..., sj] = m[..., j], l[..., j], o[..., j, :], e[..., j]
    e2[..., 10:] = 0                      # unmarked garbage beyond n_active
    out2, lse2 = oracle.merge(m2, l2, o2, e2, n_active=np.full(2, 10, np.int32))
    assert np.array_equal(out, out2) and np.array_equal(lse, lse2)


def test_merge_of_disjoint_sets_is_union():
    """Attention over a union of two disjoint cell sets = LSE merge of the two partial results."""
    pool, q, pos = small_case(63, d=64, cap=512, n_valid=512, rows=1)
    ids_a = np.array([[[0, 2, -1]] * 2], np.int32)
    ids_b = np.array([[[5, 7, -1]] * 2], np.int32)
    ids_u = np.array([[[0, 2, 5, 7]] * 2], np.int32)
    cnt2 = np.array([[2, 2]], np.int32)
    oa, la = oracle.attn(q, pos, pool, 2, ids=ids_a, counts=cnt2)
    ob, lb = oracle.attn(q, pos, pool, 2, ids=ids_b, counts=cnt2)
    ou, lu = oracle.attn(q, pos, pool, 2, ids=ids_u, counts=np.array([[4, 4]], np.int32))
    M = np.maximum(la, lb)
    wa, wb = np.exp(la - M), np.exp(lb - M)
    merged = (wa[..., None] * oa + wb[..., None] * ob) / (wa + wb)[..., None]
    np.testing.assert_allclose(merged, ou, rtol=0, atol=1e-12)


def test_all_empty_row():
    pool, q, _ = small_case(65, d=64, cap=200, n_valid=0, rows=1)
    pos = np.array([10], np.int32)
    out, lse = oracle.attn(q, pos, pool, 2)
    assert np.all(out == 0) and np.all(lse == -np.inf)
    m, l, o, e = oracle.chunk_partials(q, pos, pool, 2, 3, bpc=1)
    assert np.all(e == 1) and np.all(m == -np.inf) and np.all(l == 0)
    out2, lse2 = oracle.merge(m, l, o, e)
    assert np.all(out2 == 0) and np.all(lse2 == -np.inf)


# ---------------------------------------------------------------------------------------------------------------
# top-k
# ---------------------------------------------------------------------------------------------------------------
@pytest.mark.parametrize("width,k,levels,p_ninf", [
    (16, 8, 0, 0.0), (256, 32, 4, 0.0), (300, 64, 3, 0.3), (97, 97, 0, 0.1), (50, 80, 2, 0.0),
    (1024, 64, 0, 0.5), (33, 1, 1, 0.0), (64, 5, 0, 1.0),
])
def test_topk_equals_stable_sort(width, k, levels, p_ninf):
    s = synth.random_scores(71 + width, 6, width, levels=levels, p_ninf=p_ninf)
    ids, counts = oracle.topk(s, k)
    for r in range(6):
        exp_ids, exp_n = brute.sorted_topk([float(x) for x in s[r]], k)
        assert list(ids[r]) == exp_ids and counts[r] == exp_n


def test_topk_all_equal_takes_lowest_indices():
    s = np.zeros((2, 40))
    s[1, :7] = -np.inf
    ids, counts = oracle.topk(s, 5)
    assert list(ids[0]) == [0, 1, 2, 3, 4] and list(ids[1]) == [7, 8, 9, 10, 11]
    assert list(counts) == [5, 5]


def test_topk_negative_zero_ties_positive_zero():
    s = np.array([[0.0, -0.0, 1.0, -0.0, 0.0]])
    ids, _ = oracle.topk(s, 3)
    assert list(ids[0]) == [0, 1, 2]


# ---------------------------------------------------------------------------------------------------------------
# closed forms
# ---------------------------------------------------------------------------------------------------------------
def test_constant_v_gives_constant_output():
    pool, q, pos = small_case(81, d=128, cap=400, n_valid=333, rows=2)
    pool.v[:, :333] = 37
    pool.vs[:, :333] = np.float32(0.0125)
    out, _ = oracle.attn(q, pos, pool, 2)
    np.testing.assert_allclose(out, 37 * float(np.float32(0.0125)), rtol=1e-14, atol=0)


def test_zero_keys_give_uniform_weights():
    pool, q, pos = small_case(83, d=64, cap=400, n_valid=300, rows=2)
    pool.k[:, :300] = 0
    ids = np.array([[[1, 3, -1]] * 2] * 2, np.int32)
    counts = np.array([[2, 2], [2, 2]], np.int32)
    out, _ = oracle.attn(q, pos, pool, 2, ids=ids, counts=counts)
    V = brute.dequant(pool.v[:, :300], pool.vs[:, :300])
    for i in range(2):
        cells = [c for c in list(range(64, 128)) + list(range(192, 256)) if c <= pos[i]]
        for h in range(6):
            np.testing.assert_allclose(out[i, h], V[h // 3, cells].mean(axis=0), rtol=0, atol=1e-14)


def test_one_dominant_cell():
    pool, _, _ = small_case(85, d=64, cap=200, n_valid=200, rows=1)
    q = np.zeros((1, 6, 64), np.float32)
    q[0, :, 0] = 0.5
    pool.k[:, :200, 0] = 0
    pool.k[:, 77, 0] = 127
    pool.ks[:, 77, 0] = 2.0            # logit 127 for cell 77, 0 elsewhere
    out, _ = oracle.attn(q, np.array([199], np.int32), pool, 2)
    V = brute.dequant(pool.v[:, :200], pool.vs[:, :200])
    for h in range(6):
        np.testing.assert_allclose(out[0, h], V[h // 3, 77], rtol=1e-20, atol=1e-40)


def test_zero_query_selects_lowest_blocks_and_averages():
    pool, _, _ = small_case(87, d=64, cap=700, n_valid=650, rows=1)
    q = np.zeros((1, 6, 64), np.float32)
    pos = np.array([649], np.int32)
    nb = -(-650 // B)
    s = oracle.block_scores(q, pos, oracle.block_index(pool), 2, 650, nb)
    assert np.all(s == 0)
    ids, counts = oracle.topk(s.reshape(-1, nb), 4)
    assert np.all(ids == [0, 1, 2, 3]) and np.all(counts == 4)
    out, _ = oracle.attn(q, pos, pool, 2, ids=ids.reshape(1, 2, 4), counts=counts.reshape(1, 2))
    V = brute.dequant(pool.v[:, :650], pool.vs[:, :650])
    for h in range(6):
        np.testing.assert_allclose(out[0, h], V[h // 3, :256].mean(axis=0), rtol=0, atol=1e-14)


# ---------------------------------------------------------------------------------------------------------------
# index and scores
# ---------------------------------------------------------------------------------------------------------------
def test_block_index_is_block_mean():
    pool, _, _ = small_case(91, d=128, cap=500, n_valid=450)
    r = oracle.block_index(pool)
    np.testing.assert_allclose(r, brute.block_means(pool), rtol=0, atol=1e-14)
    r_wide = oracle.block_index(pool, n_blocks=10)       # blocks past n_valid hold zeros
    assert np.all(r_wide[:, 8:] == 0) and np.array_equal(r_wide[:, :8], r)


def test_score_identity_and_causal_eligibility():
    pool, q, pos = small_case(93, d=64, cap=500, n_valid=450, rows=3)
    pos = np.array([449, 130, 127], np.int32)
    nb = 9
    s = oracle.block_scores(q, pos, oracle.block_index(pool), 2, 450, nb + 2)
    K = brute.dequant(pool.k[:, :450], pool.ks[:, :450])
    for i in range(3):
        for g in range(2):
            for b in range(nb + 2):
                if b >= nb or b * B > pos[i]:
                    assert s[i, g, b] == -np.inf
                    continue
                cells = range(b * B, min((b + 1) * B, 450))
                per_cell = [sum(float(np.dot(q[i, h].astype(np.float64), K[g, c])) for h in range(3 * g, 3 * g + 3))
                            for c in cells]
                assert abs(s[i, g, b] - math.fsum(per_cell) / len(per_cell)) < 1e-12


def test_oracle_never_reads_poison():
    pool, q, pos = small_case(95, d=64, cap=400, n_valid=190, rows=2, poison=True)
    assert np.isnan(pool.ks[0, 190, 0])
    nb = 3
    s = oracle.block_scores(q, pos, oracle.block_index(pool), 2, 190, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), 3)
    out, lse = oracle.attn(q, pos, pool, 2, ids=ids.reshape(2, 2, 3), counts=counts.reshape(2, 2))
    assert np.all(np.isfinite(out)) and np.all(np.isfinite(lse)) and np.all(np.isfinite(s))


# ---------------------------------------------------------------------------------------------------------------
# 24-bit operand split
# ---------------------------------------------------------------------------------------------------------------
def test_split24_exact_over_whole_range():
    X = np.arange(-127 * 65536, 127 * 65536 + 1, dtype=np.int32)
    h, l, m = oracle.split24(X)
    for part in (h, l, m):
        assert part.min() >= -128 and part.max() <= 127
    rec = 65536 * h.astype(np.int64) + 256 * l.astype(np.int64) + m.astype(np.int64)
    assert np.array_equal(rec, X.astype(np.int64))


def test_quant24_error_bound():
    rng = np.random.Generator(np.random.PCG64(5))
    x = rng.standard_normal(200_000)
    amax = float(np.abs(x).max())
    X = oracle.quant24(x, amax)
    assert np.abs(X).max() <= 127 * 65536
    xs = x * 127.0 / amax
    assert np.abs(xs - X / 65536.0).max() <= 2.0 ** -17
    # round half to even at exact halves
    halves = np.array([0.5, 1.5, 2.5, -0.5, -1.5]) / 65536.0 * 1.0
    Xh = oracle.quant24(halves, 127.0)
    assert list(Xh) == [0, 2, 2, 0, -2]


# ------------------------------------------------------------------------------------------------ int8 encoder
def _f32(x):
    return np.float32(x)


@pytest.mark.parametrize("seed", range(6))
def test_encode_is_nearest_code_by_brute_force(seed):
    rng = np.random.default_rng(900 + seed)
    x = (rng.standard_normal(64) * rng.choice([1e-3, 1.0, 37.0])).astype(np.float32)
    codes, scale = oracle.encode_group(x)
    amax = np.float32(np.abs(x).max())
    inv = _f32(np.float32(127.0) / amax)
    y = (x * inv).astype(np.float32)                         # the fp32 product the code is taken from
    cand = np.arange(-127, 128, dtype=np.float64)
    dist = np.abs(y.astype(np.float64)[:, None] - cand[None, :])
    best = cand[np.argmin(dist, axis=1)]                      # nearest of the 255 codes (lower on a tie...)
    ties = np.abs(np.abs(y - np.trunc(y)) - 0.5) == 0         # ...so exact halves are checked separately: even code
    assert np.all(codes[~ties] == best[~ties])
    assert np.all(codes[ties] % 2 == 0)
    assert scale == np.float32(amax / np.float32(127.0))
    assert np.abs(codes[np.argmax(np.abs(x))]) == 127          # the largest magnitude maps to +-127
    assert np.all(np.sign(codes[codes != 0]) == np.sign(x[codes != 0]))


def test_encode_recovers_power_of_two_grids_exactly():
    rng = np.random.default_rng(910)
    for e in (-12, -3, 0, 5):
        k = rng.integers(-127, 128, 64)
        k[7] = 127 if rng.random() < 0.5 else -127               # amax = 127 * 2^e: 127 / amax = 2^-e exactly
        x = (k * 2.0 ** e).astype(np.float32)
        codes, scale = oracle.encode_group(x)
        assert np.array_equal(codes.astype(np.int64), k)
        assert scale == np.float32(2.0 ** e)


def test_encode_zero_group_and_reconstruction_bound():
    codes, scale = oracle.encode_group(np.zeros(64, np.float32))
    assert scale == 0.0 and np.all(codes == 0)
    rng = np.random.default_rng(920)
    for _ in range(20):
        x = (rng.standard_normal(64) * 3.0).astype(np.float32)
        codes, scale = oracle.encode_group(x)
        err = np.abs(x.astype(np.float64) - scale * codes.astype(np.float64))
        assert err.max() <= 0.5 * scale * (1 + 2.0 ** -20) + 1e-12 * np.abs(x).max()


def test_kv_append_touches_only_its_cells():
    pool = synth.random_pool(930, 2, 300, 290, 128, poison=False)
    rng = np.random.default_rng(931)
    kn = rng.standard_normal((3, 2, 128)).astype(np.float32)
    vn = rng.standard_normal((3, 2, 128)).astype(np.float32)
    cells = np.array([5, 289, 295], np.int32)                 # 295 >= n_valid: skipped
    out = oracle.kv_append(pool, kn, vn, cells)
    changed = np.any(out.k != pool.k, axis=-1) | np.any(out.v != pool.v, axis=-1)
    assert set(np.nonzero(changed.any(axis=0))[0]) <= {5, 289}
    assert np.array_equal(out.k[:, 295], pool.k[:, 295]) and np.array_equal(out.ks[:, 295], pool.ks[:, 295])
    for r, c in enumerate(cells[:2]):
        for g in range(2):
            for t in range(2):
                codes, scale = oracle.encode_group(kn[r, g, 64 * t:64 * t + 64])
                assert np.array_equal(out.k[g, c, 64 * t:64 * t + 64], codes) and out.ks[g, c, t] == np.float32(scale)
                codes, scale = oracle.encode_group(vn[r, g, 64 * t:64 * t + 64])
                assert np.array_equal(out.v[g, c, 64 * t:64 * t + 64], codes) and out.vs[g, c, t] == np.float32(scale)


# ------------------------------------------------------------------------------------------------------ K8V4
def k8v4_case(seed, d=128, cap=400, n_valid=330, rows=3):
    pool = synth.random_pool(seed, 2, cap, n_valid, d, poison=True, v_bits=4)
    q = synth.random_q(seed + 1, rows, 6, d)
    pos = np.array([n_valid - rows + r for r in range(rows)], np.int32)
    return pool, q, pos


@pytest.mark.parametrize("d", [128, 192, 256])
def test_k8v4_dense_and_selected_equal_textbook(d):
    """4-bit V unpacked by numpy in the brute-force path; poison (code -8, NaN scales) past n_valid stays unread."""
    pool, q, pos = k8v4_case(950 + d, d=d)
    assert pool.v.shape[-1] == d // 2
    out, _ = oracle.attn(q, pos, pool, n_kv=2)
    np.testing.assert_allclose(out, brute.textbook_attention(q, pos, pool), rtol=0, atol=1e-12)
    sel = [[{0, 3, 5}, {1, 2}], [{4}, {0, 5}], [{5, 2, 1}, {3}]]
    ids = np.full((3, 2, 3), -1, np.int32)
    counts = np.zeros((3, 2), np.int32)
    for i in range(3):
        for g in range(2):
            b = sorted(sel[i][g])
            ids[i, g, :len(b)] = b
            counts[i, g] = len(b)
    out, _ = oracle.attn(q, pos, pool, 2, ids=ids, counts=counts)
    np.testing.assert_allclose(out, brute.textbook_attention(q, pos, pool, selected_blocks=sel), rtol=0, atol=1e-12)


def test_k8v4_v_differs_from_int8_reading():
    """A plausible slip -- reading the packed bytes as int8 V -- changes the result (the pin above would see it)."""
    pool, q, pos = k8v4_case(970)
    wrong = synth.Pool(pool.k, pool.ks, np.repeat(pool.v, 2, axis=-1), pool.vs, pool.capacity, pool.n_valid, 8)
    a, _ = oracle.attn(q, pos, pool, 2)
    b, _ = oracle.attn(q, pos, wrong, 2)
    assert np.abs(a - b).max() > 1e-3


def test_encode4_is_nearest_code_and_recovers_grids():
    rng = np.random.default_rng(980)
    for _ in range(6):
        x = (rng.standard_normal(64) * rng.choice([1e-2, 1.0, 9.0])).astype(np.float32)
        codes, scale = oracle.encode_group4(x)
        amax = np.float32(np.abs(x).max())
        y = (x * np.float32(np.float32(7.0) / amax)).astype(np.float32)
        cand = np.arange(-7, 8, dtype=np.float64)
        best = cand[np.argmin(np.abs(y.astype(np.float64)[:, None] - cand[None, :]), axis=1)]
        ties = np.abs(np.abs(y - np.trunc(y)) - 0.5) == 0
        assert np.all(codes[~ties] == best[~ties]) and np.all(codes[ties] % 2 == 0)
        assert scale == np.float32(amax / np.float32(7.0))
    for e in (-5, 0, 3):
        k = rng.integers(-7, 8, 64)
        k[3] = 7
        codes, scale = oracle.encode_group4((k * 2.0 ** e).astype(np.float32))
        assert np.array_equal(codes.astype(np.int64), k) and scale == np.float32(2.0 ** e)


def test_kv_append_k8v4_packs_nibbles():
    pool = synth.random_pool(990, 2, 200, 150, 128, poison=False, v_bits=4)
    rng = np.random.default_rng(991)
    kn = rng.standard_normal((2, 2, 128)).astype(np.float32)
    vn = rng.standard_normal((2, 2, 128)).astype(np.float32)
    cells = np.array([10, 149], np.int32)
    out = oracle.kv_append(pool, kn, vn, cells)
    unpacked = brute.v_codes(out)
    for r, c in enumerate(cells):
        for g in range(2):
            for t in range(2):
                codes, scale = oracle.encode_group4(vn[r, g, 64 * t:64 * t + 64])
                assert np.array_equal(unpacked[g, c, 64 * t:64 * t + 64], codes) and out.vs[g, c, t] == np.float32(scale)
    assert np.array_equal(brute.v_codes(out)[:, 11:149], brute.v_codes(pool)[:, 11:149])
