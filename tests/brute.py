"""Independent textbook evaluations used to pin the FP64 oracle (CPU only).

Nothing here is shared with the oracle's C code: attention is evaluated as softmax(q K^T) V over an explicit mask,
with the grouped-query mapping written as a head repeat of the KV tensors, dequantisation as a scale repeat over
each 64-dim group, and selection through Python's stable ``sorted``.
"""
import math

import numpy as np

GROUP = 64
BLOCK = 64


def dequant(codes, scales):
    """[n_kv][cap][d] float64 = codes * scale of the code's 64-dim group."""
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), GROUP, axis=-1)


def v_codes(pool):
    """V codes [n_kv][cap][d] as int8: the stored array, or the two signed nibbles of each byte of a K8V4 pool
    (low nibble = even dim), unpacked here with numpy bit operations."""
    if getattr(pool, "v_bits", 8) != 4:
        return pool.v
    b = pool.v.view(np.uint8)
    lo = (b & 0x0F).astype(np.int16)
    hi = (b >> 4).astype(np.int16)
    lo = np.where(lo >= 8, lo - 16, lo)
    hi = np.where(hi >= 8, hi - 16, hi)
    out = np.empty(b.shape[:-1] + (2 * b.shape[-1],), np.int8)
    out[..., 0::2] = lo
    out[..., 1::2] = hi
    return out


def repeat_kv(x, n_q_heads):
    """[n_kv][...] -> [n_q_heads][...]: q head h reads KV head h // (n_q_heads // n_kv)."""
    return np.repeat(x, n_q_heads // x.shape[0], axis=0)


def textbook_attention(q, pos, pool, selected_blocks=None, sm_scale=1.0):
    """out [n_rows][Hq][d] with pure-Python softmax per (row, head).

    ``selected_blocks[i][g]`` is a collection of block ids (None = every block)."""
    n_rows, n_qh, d = q.shape
    n_kv = pool.k.shape[0]
    K = repeat_kv(dequant(pool.k[:, :pool.n_valid], pool.ks[:, :pool.n_valid]), n_qh)
    V = repeat_kv(dequant(v_codes(pool)[:, :pool.n_valid], pool.vs[:, :pool.n_valid]), n_qh)
    G = n_qh // n_kv
    out = np.zeros((n_rows, n_qh, d))
    for i in range(n_rows):
        for h in range(n_qh):
            cells = []
            for c in range(pool.n_valid):
                if c > pos[i]:
                    continue
                if selected_blocks is not None and (c // BLOCK) not in selected_blocks[i][h // G]:
                    continue
                cells.append(c)
            if not cells:
                continue
            logits = [sm_scale * float(np.dot(q[i, h].astype(np.float64), K[h, c])) for c in cells]
            mx = max(logits)
            w = [math.exp(t - mx) for t in logits]
            tot = math.fsum(w)
            for e in range(d):
                out[i, h, e] = math.fsum(wj * V[h, c, e] for wj, c in zip(w, cells)) / tot
    return out


def matrix_attention(q, pos, pool, sm_scale=1.0):
    """Dense causal attention as masked matrix products (numpy float64), for medium sizes."""
    n_rows, n_qh, d = q.shape
    K = repeat_kv(dequant(pool.k[:, :pool.n_valid], pool.ks[:, :pool.n_valid]), n_qh)   # [Hq][n][d]
    V = repeat_kv(dequant(v_codes(pool)[:, :pool.n_valid], pool.vs[:, :pool.n_valid]), n_qh)
    Q = q.astype(np.float64).transpose(1, 0, 2)                                           # [Hq][rows][d]
    S = sm_scale * np.matmul(Q, K.transpose(0, 2, 1))                                     # [Hq][rows][n]
    mask = np.arange(pool.n_valid)[None, :] <= np.asarray(pos)[:, None]                   # [rows][n]
    S = np.where(mask[None], S, -np.inf)
    S = S - S.max(axis=-1, keepdims=True)
    P = np.exp(S)
    P /= P.sum(axis=-1, keepdims=True)
    return np.matmul(P, V).transpose(1, 0, 2)


def sorted_topk(row, k):
    """Top-k of one score row by Python's stable sort: keys (-score) with the original index order kept for ties."""
    elig = [(b, s) for b, s in enumerate(row) if s != -math.inf]
    ranked = sorted(elig, key=lambda bs: -bs[1])       # stable: equal scores keep ascending index
    take = sorted(b for b, _ in ranked[:k])
    return take + [-1] * (k - len(take)), len(take)


def block_means(pool):
    """[n_kv][n_blocks][d]: mean dequantised key per block, by reshaping the valid cells."""
    n_kv, cap, d = pool.k.shape
    nb = -(-pool.n_valid // BLOCK)
    K = dequant(pool.k[:, :pool.n_valid], pool.ks[:, :pool.n_valid])
    out = np.zeros((n_kv, nb, d))
    for b in range(nb):
        out[:, b] = K[:, b * BLOCK:min((b + 1) * BLOCK, pool.n_valid)].mean(axis=1)
    return out
