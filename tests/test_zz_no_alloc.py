"""qsa_decode_layer_noalloc (the decode layer over the library's per-device static scratch, for callers that cannot
allocate) against qsa_decode_layer with a caller's scratch buffer, through the C ABI: two calls in a row, the second
with a smaller input, must give the same scores, ids, counts, output and lse bits as the scratch-buffer call, and
the first also matches the FP64 oracle end to end."""
import numpy as np
import pytest
import torch

import sparse_top_attention_amd as qsa
import synth
from gpu_util import BLOCK, build_index, dev, to_device
from test_gpu_decode import _check_end_to_end, dims_of, small_workload

pytestmark = pytest.mark.gpu


def _run(fn, w, pdevs, dims, n_chunks, row_pool=None):
    n_rows = w.q.shape[0]
    nb = -(-w.pools[0].n_valid // BLOCK)
    res = dict(out=torch.full((n_rows, dims.n_q_heads, dims.head_dim), float("nan"), device="cuda"),
               lse=torch.full((n_rows, dims.n_q_heads), float("nan"), device="cuda"),
               scores=torch.full((n_rows, dims.n_kv_heads, nb), float("nan"), device="cuda"),
               ids=torch.full((n_rows, dims.n_kv_heads, w.topk), -7, dtype=torch.int32, device="cuda"),
               counts=torch.full((n_rows, dims.n_kv_heads), -7, dtype=torch.int32, device="cuda"))
    kw = dict(lse=res["lse"], sm_scale=w.sm_scale, row_pool=row_pool, scores=res["scores"], ids=res["ids"],
              counts=res["counts"])
    if fn == "noalloc":
        qsa.qsa_decode_layer_noalloc(dev(w.q), dev(w.pos), pdevs, dims, nb, w.topk, n_chunks, res["out"], **kw)
    else:
        scratch = torch.empty(qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, nb, w.topk, n_chunks),
                              dtype=torch.uint8, device="cuda")
        qsa.qsa_decode_layer(dev(w.q), dev(w.pos), pdevs, dims, nb, w.topk, n_chunks, res["out"], scratch=scratch,
                             **kw)
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in res.items()}


def _same(a, b):
    for key in ("scores", "ids", "counts", "out", "lse"):
        assert np.array_equal(a[key], b[key]), key


def test_noalloc_matches_scratch_call_twice_then_smaller():
    # 1: the verify window at full size (200,000-cell pool, 16 chunks)
    w = synth.workload("verify_window")
    dims = dims_of(w)
    p = build_index(to_device(w.pools[0]), dims)
    first = _run("noalloc", w, [p], dims, 16)
    _same(first, _run("scratch", w, [p], dims, 16))
    _check_end_to_end(w, first)
    # 2: right after it, a smaller layer (3 rows, 2 KV heads, 5 chunks) over the same static array
    w2 = small_workload(1301, n_kv=2, G=6, rows=3, topk=9)
    dims2 = dims_of(w2)
    p2 = build_index(to_device(w2.pools[0]), dims2)
    second = _run("noalloc", w2, [p2], dims2, 5)
    _same(second, _run("scratch", w2, [p2], dims2, 5))
    _check_end_to_end(w2, second)


def test_noalloc_two_pools_and_limit():
    w = synth.workload("batch_window")
    dims = dims_of(w)
    pdevs = [build_index(to_device(pl), dims) for pl in w.pools]
    rp = dev(w.row_pool)
    _same(_run("noalloc", w, pdevs, dims, 32, row_pool=rp), _run("scratch", w, pdevs, dims, 32, row_pool=rp))
    # a layer whose scratch exceeds the static array is refused with QSA_ERR_SCRATCH before any launch
    nb = -(-w.pools[0].n_valid // BLOCK)
    n_rows = 64
    assert qsa.qsa_decode_layer_scratch_bytes(n_rows, dims, nb, w.topk, 64) > qsa.NOALLOC_SCRATCH_BYTES
    q = torch.zeros(n_rows, dims.n_q_heads, dims.head_dim, device="cuda")
    pos = torch.zeros(n_rows, dtype=torch.int32, device="cuda")
    out = torch.full((n_rows, dims.n_q_heads, dims.head_dim), 3.0, device="cuda")
    with pytest.raises(qsa.QSAError) as e:
        qsa.qsa_decode_layer_noalloc(q, pos, pdevs[:1], dims, nb, w.topk, 64, out)
    assert e.value.status == -4
    torch.cuda.synchronize()
    assert bool((out == 3.0).all())
