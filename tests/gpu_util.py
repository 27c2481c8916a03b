"""GPU-side helpers for the parity tests: move synthetic workloads to the device and run the decode path through
the C ABI. Comparisons are made against the FP64 oracle in the tests themselves."""
import numpy as np
import torch

import sparse_top_attention_amd as qsa

BLOCK = 64


def dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def to_device(pool):
    """synth.Pool (numpy) -> qsa.Pool on the GPU, with a block-index buffer allocated (not yet filled)."""
    n_kv, cap, d = pool.k.shape
    p = qsa.Pool(dev(pool.k), dev(pool.ks), dev(pool.v), dev(pool.vs), pool.n_valid, v_bits=pool.v_bits)
    p.index = torch.full((n_kv, -(-cap // BLOCK), d), float("nan"), dtype=torch.float32, device="cuda")
    return p


def build_index(p, dims):
    qsa.qsa_block_index(p, dims, 0, p.n_valid, p.index)
    return p


def rel_err_rows(x, ref):
    """Per (row, head) error max_d |x - ref| / max_d |ref| (ref all-zero rows: max |x|)."""
    x = np.asarray(x, np.float64)
    ref = np.asarray(ref, np.float64)
    num = np.abs(x - ref).max(axis=-1)
    den = np.abs(ref).max(axis=-1)
    return np.where(den > 0, num / np.where(den > 0, den, 1), num)


def score_errors(s_gpu, s_ref, qt_abs_r):
    """Score error relative to sum_d |qsum_d r_d| of each entry; -inf must match exactly."""
    ninf_gpu = np.isneginf(s_gpu)
    ninf_ref = np.isneginf(s_ref)
    assert np.array_equal(ninf_gpu, ninf_ref), "ineligible blocks differ"
    fin = ~ninf_ref
    err = np.zeros_like(s_ref)
    err[fin] = np.abs(s_gpu[fin] - s_ref[fin]) / np.maximum(qt_abs_r[fin], 1e-30)
    return err


def qsum_abs_dot(q, r, G):
    """sum_d |qsum_d r_{g,b,d}| for every (row, KV head, block): the scale of a score's rounding error."""
    n_rows, n_qh, d = q.shape
    n_kv = n_qh // G
    qt = q.astype(np.float64).reshape(n_rows, n_kv, G, d).sum(axis=2)          # [rows][kv][d]
    return np.einsum("igd,gbd->igb", np.abs(qt), np.abs(r.astype(np.float64)))


def topk_margin_ok(s_ref, k, scale, tol=1e-5):
    """Rows whose k-th and (k+1)-th eligible FP64 scores are further apart than tol * max scale of the row."""
    R, W = s_ref.shape
    ok = np.ones(R, bool)
    for r in range(R):
        fin = np.sort(s_ref[r][np.isfinite(s_ref[r])])[::-1]
        if len(fin) <= k:
            continue
        margin = fin[k - 1] - fin[k]
        ok[r] = margin > tol * scale[r].max()
    return ok


def decode_layer(w, p_dev, dims, n_chunks, ids_override=None, nb=None):
    """scores -> topk -> chunk -> merge for a one-pool workload (score rows of nb columns, default the valid
    blocks); returns a dict of host arrays."""
    pool = p_dev
    n_rows = w.q.shape[0]
    nb = nb or -(-w.pools[0].n_valid // BLOCK)
    q = dev(w.q)
    pos = dev(w.pos)
    scores = torch.empty(n_rows, dims.n_kv_heads, nb, dtype=torch.float32, device="cuda")
    qsa.qsa_block_scores(q, pos, pool, dims, nb, scores)
    ids = torch.empty(n_rows, dims.n_kv_heads, w.topk, dtype=torch.int32, device="cuda")
    counts = torch.empty(n_rows, dims.n_kv_heads, dtype=torch.int32, device="cuda")
    qsa.qsa_topk(scores, w.topk, ids, counts)
    if ids_override is not None:
        ids = dev(ids_override[0])
        counts = dev(ids_override[1])
    part = qsa.Partials.empty_like_shape(n_rows, dims.n_q_heads, n_chunks, dims.head_dim)
    qsa.qsa_attn_chunk(q, pos, [pool], dims, part, n_chunks, w.sm_scale, ids=ids, counts=counts)
    out = torch.empty(n_rows, dims.n_q_heads, dims.head_dim, dtype=torch.float32, device="cuda")
    lse = torch.empty(n_rows, dims.n_q_heads, dtype=torch.float32, device="cuda")
    qsa.qsa_attn_merge(part, dims, n_chunks, out, lse)
    torch.cuda.synchronize()
    return dict(scores=scores.cpu().numpy(), ids=ids.cpu().numpy(), counts=counts.cpu().numpy(),
                m=part.m.cpu().numpy(), l=part.l.cpu().numpy(), o=part.o.cpu().numpy(),
                empty=part.empty.cpu().numpy(), out=out.cpu().numpy(), lse=lse.cpu().numpy(),
                index=pool.index.cpu().numpy())
