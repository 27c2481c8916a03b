"""Every error path of the C ABI returns its status before any launch: called on the GPU with real device buffers that
hold a canary pattern, each rejected call must leave every output buffer untouched. Calls go straight to the C ABI
(the binding's own size checks would stop most of these earlier)."""
import ctypes

import numpy as np
import pytest
import torch

import sparse_top_attention_amd as qsa
import synth
from gpu_util import BLOCK, build_index, dev, to_device

pytestmark = pytest.mark.gpu
CANARY = 1234.5


def _canary(*shape, dtype=torch.float32):
    if dtype == torch.float32:
        return torch.full(shape, CANARY, dtype=dtype, device="cuda")
    return torch.full(shape, 77, dtype=dtype, device="cuda")


def _unchanged(*tensors):
    torch.cuda.synchronize()
    for t in tensors:
        ref = CANARY if t.dtype == torch.float32 else 77
        assert bool((t == ref).all()), "a rejected call wrote to an output"


@pytest.fixture(scope="module")
def setup():
    w = synth.workload("tiny_decode")
    dims = qsa.Dims(w.n_q_heads, w.n_kv_heads, w.head_dim)
    p = build_index(to_device(w.pools[0]), dims)
    torch.cuda.synchronize()
    return w, dims, p


def _ptr(t):
    return None if t is None else t.data_ptr()


def test_rejected_calls_write_nothing(setup):
    w, dims, p = setup
    L = qsa.lib_handle()
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    pc = p.c()
    pools = (qsa._Pool * 1)(pc)
    D, Hq, Hkv = dims.head_dim, dims.n_q_heads, dims.n_kv_heads
    q, pos = dev(w.q), dev(w.pos)
    nb = -(-w.pools[0].n_valid // BLOCK)
    bad_dims = qsa._Dims(Hq, Hkv, 320, 64)

    # block index: cell range past the capacity (QSA_ERR_RANGE); head_dim 320 (QSA_ERR_UNSUPPORTED)
    index = _canary(*p.index.shape)
    assert L.qsa_block_index(ctypes.byref(pc), dims.c(), 0, p.capacity + 1, _ptr(index), s) == -5
    assert L.qsa_block_index(ctypes.byref(pc), bad_dims, 0, 64, _ptr(index), s) == -3
    _unchanged(index)

    # block scores: rows wider than the capacity's blocks (QSA_ERR_RANGE)
    scores = _canary(1, Hkv, nb + 1)
    too_wide = -(-p.capacity // BLOCK) + 1
    assert L.qsa_block_scores(_ptr(q), _ptr(pos), 1, ctypes.byref(pc), dims.c(), too_wide, _ptr(scores), s) == -5
    _unchanged(scores)

    # top-k: k past the row width (QSA_ERR_RANGE), width past 16,384 (QSA_ERR_UNSUPPORTED or RANGE)
    srows = dev(synth.random_scores(5, 4, 16))
    ids, counts = _canary(4, 32, dtype=torch.int32), _canary(4, dtype=torch.int32)
    assert L.qsa_topk(_ptr(srows), 4, 16, 17, _ptr(ids), _ptr(counts), None, 0, s) == -5
    assert L.qsa_topk(_ptr(srows), 4, 16, 0, _ptr(ids), _ptr(counts), None, 0, s) == -5
    _unchanged(ids, counts)

    # chunk attention: more chunks than the partials hold (QSA_ERR_SCRATCH); zero chunks (QSA_ERR_RANGE)
    part = qsa.Partials(_canary(1, Hq, 4), _canary(1, Hq, 4), _canary(1, Hq, 4, D), _canary(1, Hq, 4, dtype=torch.uint8))
    parts = part.c()
    for n_chunks, code in ((5, -4), (0, -5)):
        assert L.qsa_attn_chunk(_ptr(q), _ptr(pos), 1, pools, 1, None, dims.c(), None, None, 0, 1, n_chunks, 1.0,
                                ctypes.byref(parts), s) == code
    _unchanged(part.m, part.l, part.o, part.empty)

    # merge: zero chunks (QSA_ERR_RANGE), more than the partials hold (QSA_ERR_SCRATCH)
    out, lse = _canary(1, Hq, D), _canary(1, Hq)
    assert L.qsa_attn_merge(ctypes.byref(parts), 1, dims.c(), 0, None, _ptr(out), _ptr(lse), s) == -5
    assert L.qsa_attn_merge(ctypes.byref(parts), 1, dims.c(), 5, None, _ptr(out), _ptr(lse), s) == -4
    _unchanged(out, lse)

    # one-launch selection: k = 0 (QSA_ERR_RANGE)
    sel_ids, sel_cnt = _canary(1, Hkv, 8, dtype=torch.int32), _canary(1, Hkv, dtype=torch.int32)
    assert L.qsa_decode_select(_ptr(q), _ptr(pos), 1, pools, 1, None, dims.c(), nb, 0, None, _ptr(sel_ids),
                               _ptr(sel_cnt), s) == -5
    _unchanged(sel_ids, sel_cnt)

    # decode layer: scratch one byte short (QSA_ERR_SCRATCH), k past the width (QSA_ERR_RANGE)
    need = L.qsa_decode_layer_scratch_bytes(1, dims.c(), nb, w.topk, 4)
    scratch = torch.full((need,), 77, dtype=torch.uint8, device="cuda")
    assert L.qsa_decode_layer(_ptr(q), _ptr(pos), 1, pools, 1, None, dims.c(), nb, w.topk, 4, 1.0, _ptr(out),
                              _ptr(lse), None, None, None, _ptr(scratch), need - 1, s) == -4
    assert L.qsa_decode_layer(_ptr(q), _ptr(pos), 1, pools, 1, None, dims.c(), nb, nb + 1, 4, 1.0, _ptr(out),
                              _ptr(lse), None, None, None, _ptr(scratch), need, s) == -5
    _unchanged(out, lse, scratch)

    # prompt: scratch one byte short (QSA_ERR_SCRATCH); head_dim 320 (QSA_ERR_UNSUPPORTED)
    pq = dev(synth.random_q(9, 8, Hq, D))
    pout = _canary(8, Hq, D)
    pneed = L.qsa_prompt_scratch_bytes(8, 100, dims.c())
    pscr = torch.full((pneed,), 77, dtype=torch.uint8, device="cuda")
    assert L.qsa_prompt_attn(_ptr(pq), 8, 100, ctypes.byref(pc), dims.c(), 1.0, _ptr(pout), _ptr(pscr), pneed - 1,
                             s) == -4
    assert L.qsa_prompt_attn(_ptr(pq), 8, 100, ctypes.byref(pc), bad_dims, 1.0, _ptr(pout), _ptr(pscr), pneed,
                             s) == -3
    _unchanged(pout, pscr)

    # append: unsupported head_dim, then a pool whose n_valid exceeds its capacity (QSA_ERR_RANGE)
    k_new = dev(np.ones((1, Hkv, D), np.float32))
    cells = dev(np.array([5], np.int32))
    before = p.k.clone(), p.k_scale.clone(), p.v.clone(), p.v_scale.clone(), p.index.clone()
    assert L.qsa_kv_append(pools, 1, None, bad_dims, _ptr(k_new), _ptr(k_new), _ptr(cells), 1, s) == -3
    bad_pool = qsa._Pool(pc.k, pc.k_scale, pc.v, pc.v_scale, pc.index, pc.capacity, pc.capacity + 1, 8)
    assert L.qsa_kv_append((qsa._Pool * 1)(bad_pool), 1, None, dims.c(), _ptr(k_new), _ptr(k_new), _ptr(cells), 1,
                           s) == -5
    torch.cuda.synchronize()
    for a, b in zip(before, (p.k, p.k_scale, p.v, p.v_scale, p.index)):
        assert torch.equal(a, b)
