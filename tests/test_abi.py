"""The C-ABI library (CPU only): it loads, exports every function include/qsa.h declares, and its host-side
argument checks return the documented status codes. These calls fail validation before any HIP call, so no
GPU is touched."""
import ctypes
import os
import re

import pytest

import sparse_top_attention_amd as qsa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "qsa.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\**\s*(qsa_[a-z0-9_]+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_the_calls():
    names = declared_functions()
    for fn in ["qsa_block_index", "qsa_block_scores", "qsa_topk", "qsa_topk_scratch_bytes", "qsa_attn_chunk",
               "qsa_attn_merge", "qsa_prompt_attn", "qsa_prompt_scratch_bytes", "qsa_decode_layer",
               "qsa_decode_layer_scratch_bytes", "qsa_decode_select", "qsa_kv_append", "qsa_status_str",
               "qsa_decode_layer_noalloc"]:
        assert fn in names


def test_library_exports_every_declared_symbol():
    L = qsa.lib_handle()
    for fn in declared_functions():
        assert hasattr(L, fn), fn


def test_no_symbol_from_the_oracle():
    L = ctypes.CDLL(qsa.LIB_PATH)
    for fn in ["orc_attn", "orc_topk", "orc_merge", "orc_block_scores"]:
        assert not hasattr(L, fn)


def test_status_strings():
    for code in range(-6, 1):
        assert qsa.qsa_status_str(code)


D = qsa._Dims


def _pool(k=1, ks=1, v=1, vs=1, index=1, cap=1024, n_valid=1024, v_bits=8):
    return qsa._Pool(k, ks, v, vs, index, cap, n_valid, v_bits)


def _parts(max_chunks=8):
    return qsa._Partials(1, 1, 1, 1, max_chunks)


GOOD = D(24, 4, 128, 64)


@pytest.mark.parametrize("dims,expect", [
    (D(24, 4, 96, 64), -3),    # head_dim not supported
    (D(24, 4, 320, 64), -3),   # 64-dim groups, but past 256
    (D(24, 4, 128, 32), -3),   # block size not 64
    (D(24, 5, 128, 64), -2),   # q heads not a multiple of KV heads
    (D(40, 4, 128, 64), -3),   # more than 8 q heads per KV head
    (D(0, 4, 128, 64), -2),
    (D(65536, 65536, 128, 64), -3),   # KV heads past a launch grid dimension
])
def test_dims_validation(dims, expect):
    L = qsa.lib_handle()
    p = _pool()
    assert L.qsa_block_index(ctypes.byref(p), dims, 0, 64, 1, None) == expect
    assert L.qsa_block_scores(1, 1, 1, ctypes.byref(p), dims, 16, 1, None) == expect


def test_block_index_validation():
    L = qsa.lib_handle()
    assert L.qsa_block_index(None, GOOD, 0, 64, 1, None) == -1
    p = _pool()
    assert L.qsa_block_index(ctypes.byref(p), GOOD, 0, 64, None, None) == -1
    assert L.qsa_block_index(ctypes.byref(p), GOOD, -1, 64, 1, None) == -5
    assert L.qsa_block_index(ctypes.byref(p), GOOD, 100, 64, 1, None) == -5
    assert L.qsa_block_index(ctypes.byref(p), GOOD, 0, 2000, 1, None) == -5
    assert L.qsa_block_index(ctypes.byref(p), GOOD, 64, 64, 1, None) == 0      # empty range: nothing to do
    bad = _pool(n_valid=2000)
    assert L.qsa_block_index(ctypes.byref(bad), GOOD, 0, 64, 1, None) == -5    # n_valid > capacity
    nok = _pool(k=None)
    assert L.qsa_block_index(ctypes.byref(nok), GOOD, 0, 64, 1, None) == -1


def test_block_scores_validation():
    L = qsa.lib_handle()
    p = _pool()
    assert L.qsa_block_scores(None, 1, 1, ctypes.byref(p), GOOD, 16, 1, None) == -1
    noidx = _pool(index=None)
    assert L.qsa_block_scores(1, 1, 1, ctypes.byref(noidx), GOOD, 16, 1, None) == -1
    assert L.qsa_block_scores(1, 1, 1, ctypes.byref(p), GOOD, 17, 1, None) == -5  # wider than ceil(cap/64)
    assert L.qsa_block_scores(1, 1, -1, ctypes.byref(p), GOOD, 16, 1, None) == -2
    assert L.qsa_block_scores(1, 1, 0, ctypes.byref(p), GOOD, 16, 1, None) == 0    # no rows: nothing to do


def test_topk_validation():
    L = qsa.lib_handle()
    assert L.qsa_topk_scratch_bytes(16, 256, 32) == 0
    assert L.qsa_topk(None, 1, 16, 8, 1, 1, None, 0, None) == -1
    assert L.qsa_topk(1, 1, 16, 0, 1, 1, None, 0, None) == -5
    assert L.qsa_topk(1, 1, 16, 17, 1, 1, None, 0, None) == -5
    assert L.qsa_topk(1, 1, 20000, 8, 1, 1, None, 0, None) == -3
    assert L.qsa_topk(1, 0, 16, 8, 1, 1, None, 0, None) == 0


def test_chunk_validation():
    L = qsa.lib_handle()
    pools = (qsa._Pool * 2)(_pool(), _pool())
    parts = _parts(8)
    args = dict(q=1, pos=1, n_rows=4, pools=pools, n_pools=2, row_pool=1, dims=GOOD, ids=1, counts=1, k=32,
                bpc=1, n_chunks=8, sm=1.0, out=ctypes.byref(parts), stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.qsa_attn_chunk(a["q"], a["pos"], a["n_rows"], a["pools"], a["n_pools"], a["row_pool"], a["dims"],
                                a["ids"], a["counts"], a["k"], a["bpc"], a["n_chunks"], a["sm"], a["out"],
                                a["stream"])
    assert call(n_chunks=9) == -4                        # partials too small
    for bad in (float("inf"), float("-inf"), float("nan")):   # any finite scale is taken, negative included
        assert call(sm=bad) == -5
    assert call(n_chunks=0) == -5
    assert call(k=0) == -5
    assert call(counts=None) == -1
    assert call(q=None) == -1
    assert call(n_pools=9) == -3
    assert call(n_pools=0) == -2
    assert call(ids=None, bpc=0) == -5
    bad = (qsa._Pool * 2)(_pool(), _pool(n_valid=5000))
    assert call(pools=bad) == -5
    nov = (qsa._Pool * 1)(_pool(v=None))
    assert call(pools=nov, n_pools=1) == -1
    noparts = qsa._Partials(1, None, 1, 1, 8)
    assert call(out=ctypes.byref(noparts)) == -1
    assert call(n_rows=0) == 0


def test_merge_validation():
    L = qsa.lib_handle()
    parts = _parts(8)
    assert L.qsa_attn_merge(ctypes.byref(parts), 4, GOOD, 9, None, 1, None, None) == -4
    assert L.qsa_attn_merge(None, 4, GOOD, 8, None, 1, None, None) == -1
    assert L.qsa_attn_merge(ctypes.byref(parts), 4, GOOD, 8, None, None, None, None) == -1
    assert L.qsa_attn_merge(ctypes.byref(parts), 0, GOOD, 8, None, 1, None, None) == 0
    # no chunks to fold: refused before any launch (the kernel's clamp target would be chunk -1)
    assert L.qsa_attn_merge(ctypes.byref(parts), 4, GOOD, 0, None, 1, None, None) == -5
    assert L.qsa_attn_merge(ctypes.byref(parts), 0, GOOD, 0, None, 1, None, None) == -5
    assert L.qsa_attn_merge(ctypes.byref(parts), 4, GOOD, -1, None, 1, None, None) == -5
    # one workgroup per (row, q head): more than INT32_MAX of them is refused, not launched on a wrapped grid
    assert L.qsa_attn_merge(ctypes.byref(parts), 2**27, GOOD, 8, None, 1, None, None) == -3


def test_prompt_validation():
    L = qsa.lib_handle()
    p = _pool()
    assert L.qsa_prompt_attn(None, 16, 0, ctypes.byref(p), GOOD, 1.0, 1, None, 0, None) == -1
    assert L.qsa_prompt_attn(1, 16, -1, ctypes.byref(p), GOOD, 1.0, 1, None, 0, None) == -5
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p), GOOD, float("inf"), 1, None, 0, None) == -5
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p), D(24, 4, 96, 64), 1.0, 1, None, 0, None) == -3


def test_prompt_scratch_sizing_and_checks():
    L = qsa.lib_handle()
    n = L.qsa_prompt_scratch_bytes(2048, 30720, GOOD)
    assert n >= 2048 * 24 * (3 * 128 + 4)          # q digits and row scales at least
    assert n >= 2048 * 24 * 2 * (128 * 4 + 9)      # and two cell chunks' (m, l, empty, o) partials per row
    # a handful of queries is split into many more cell chunks, so its few row blocks spread over the chip
    assert L.qsa_prompt_scratch_bytes(16, 4096, GOOD) >= 16 * 24 * 16 * (128 * 4 + 9)
    assert L.qsa_prompt_scratch_bytes(0, 0, GOOD) == 0
    assert L.qsa_prompt_scratch_bytes(16, -1, GOOD) == 0
    assert L.qsa_prompt_scratch_bytes(2**27, 0, GOOD) == 0     # more (query, head) rows than an int32 holds
    # head_dims without the int8 matrix-core kernel take the dense chunk path: its partials for one 64-query batch
    d64, d256 = D(24, 4, 64, 64), D(24, 4, 256, 64)
    assert L.qsa_prompt_scratch_bytes(16, 0, d64) >= 16 * 24 * 1 * (64 * 4 + 9)
    assert L.qsa_prompt_scratch_bytes(100, 4000, d256) >= 64 * 24 * 32 * (256 * 4 + 9)
    d192 = D(24, 4, 192, 64)
    assert L.qsa_prompt_scratch_bytes(16, 0, d192) >= 16 * 24 * 1 * (192 * 4 + 9)
    p = _pool()
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p), GOOD, 1.0, 1, None, 0, None) == -1       # no scratch
    need = L.qsa_prompt_scratch_bytes(16, 0, GOOD)
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p), GOOD, 1.0, 1, 1, need - 1, None) == -4
    # the dense path checks its own scratch need; a K8V4 pool at head_dim 128 needs the matrix-core kernel's
    need64 = L.qsa_prompt_scratch_bytes(16, 0, d64)
    p64 = _pool()
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p64), d64, 1.0, 1, 1, need64 - 1, None) == -4
    p4 = _pool(v_bits=4)
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p4), GOOD, 1.0, 1, 1, 0, None) == -4
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p4), d64, 1.0, 1, 1, need, None) == -3     # K8V4 at head_dim 64
    need192 = L.qsa_prompt_scratch_bytes(16, 0, d192)
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p), d192, 1.0, 1, 1, need192 - 1, None) == -4
    assert L.qsa_prompt_attn(1, 2, 2**31 - 1, ctypes.byref(p), GOOD, 1.0, 1, 1, need, None) == -5  # positions past int32
    assert L.qsa_prompt_attn(1, 2**27, 0, ctypes.byref(p), GOOD, 1.0, 1, 1, need, None) == -3  # 3.2e9 (query, head) rows
    assert L.qsa_prompt_attn(1, 0, 0, ctypes.byref(p), GOOD, 1.0, 1, None, 0, None) == 0


def test_decode_layer_validation():
    L = qsa.lib_handle()
    pools = (qsa._Pool * 2)(_pool(), _pool())
    need = L.qsa_decode_layer_scratch_bytes(4, GOOD, 16, 8, 4)
    assert need >= 4 * 24 * 4 * (128 * 4 + 9)             # the partials at least
    assert need >= 4 * 24 * 4 * (128 * 4 + 9) + 4 * 4 * 16 * 4   # and the score rows of 16 columns
    assert L.qsa_decode_layer_scratch_bytes(4, GOOD, 1024, 8, 4) >= need + 4 * 4 * (1024 - 16) * 4 - 256
    assert L.qsa_decode_layer_scratch_bytes(0, GOOD, 16, 8, 4) == 0
    assert L.qsa_decode_layer_scratch_bytes(4, GOOD, 16, 0, 4) == 0
    assert L.qsa_decode_layer_scratch_bytes(4, GOOD, 0, 8, 4) == 0
    args = dict(q=1, pos=1, n_rows=4, pools=pools, n_pools=2, row_pool=1, dims=GOOD, nb=16, k=8, S=4, sm=1.0,
                out=1, lse=None, scores=None, ids=None, counts=None, scratch=1, nbytes=need, stream=None)

    def call(**kw):
        a = dict(args)
        a.update(kw)
        return L.qsa_decode_layer(a["q"], a["pos"], a["n_rows"], a["pools"], a["n_pools"], a["row_pool"],
                                  a["dims"], a["nb"], a["k"], a["S"], a["sm"], a["out"], a["lse"], a["scores"],
                                  a["ids"], a["counts"], a["scratch"], a["nbytes"], a["stream"])
    assert call(q=None) == -1
    assert call(out=None) == -1
    assert call(scratch=None) == -1
    assert call(nbytes=need - 1) == -4
    assert call(k=0) == -5
    assert call(k=17) == -5                                # k > n_blocks
    assert call(nb=17) == -5                               # wider than ceil(cap / 64)
    assert call(S=0) == -5
    assert call(sm=float("nan")) == -5
    assert call(sm=float("inf")) == -5
    assert call(n_pools=9) == -3
    assert call(dims=D(24, 4, 96, 64)) == -3
    noidx = (qsa._Pool * 2)(_pool(), _pool(index=None))
    assert call(pools=noidx) == -1
    assert call(n_rows=0) == 0


def test_decode_select_validation():
    L = qsa.lib_handle()
    pools = (qsa._Pool * 1)(_pool())
    assert L.qsa_decode_select(1, 1, 4, pools, 1, None, GOOD, 16, 8, None, None, 1, None) == -1   # ids required
    assert L.qsa_decode_select(1, 1, 4, pools, 1, None, GOOD, 16, 8, None, 1, None, None) == -1   # counts required
    assert L.qsa_decode_select(1, 1, 4, pools, 1, None, GOOD, 16, 0, None, 1, 1, None) == -5
    assert L.qsa_decode_select(1, 1, 4, pools, 1, None, GOOD, 17, 8, None, 1, 1, None) == -5
    assert L.qsa_decode_select(1, 1, 0, pools, 1, None, GOOD, 16, 8, None, 1, 1, None) == 0


def test_kv_append_validation():
    L = qsa.lib_handle()
    pools = (qsa._Pool * 2)(_pool(), _pool())
    assert L.qsa_kv_append(pools, 2, 1, GOOD, None, 1, 1, 4, None) == -1
    assert L.qsa_kv_append(pools, 2, 1, GOOD, 1, 1, None, 4, None) == -1
    assert L.qsa_kv_append(pools, 9, 1, GOOD, 1, 1, 1, 4, None) == -3
    assert L.qsa_kv_append(pools, 2, 1, D(24, 4, 96, 64), 1, 1, 1, 4, None) == -3
    assert L.qsa_kv_append(pools, 2, 1, GOOD, 1, 1, 1, -1, None) == -2
    bad = (qsa._Pool * 1)(_pool(n_valid=2000))
    assert L.qsa_kv_append(bad, 1, None, GOOD, 1, 1, 1, 4, None) == -5
    assert L.qsa_kv_append(pools, 2, 1, GOOD, 1, 1, 1, 0, None) == 0


def test_v_bits_validation():
    """V formats: 0/8 int8, 4 K8V4; anything else, mixed formats in one call and K8V4 at head_dim 64 (in the decode
    calls and in the prompt call) are unsupported."""
    L = qsa.lib_handle()
    parts = _parts(8)

    def chunk(pools, n, dims=GOOD):
        return L.qsa_attn_chunk(1, 1, 4, pools, n, 1, dims, 1, 1, 32, 1, 8, 1.0, ctypes.byref(parts), None)
    assert chunk((qsa._Pool * 1)(_pool(v_bits=3)), 1) == -3
    assert chunk((qsa._Pool * 2)(_pool(v_bits=8), _pool(v_bits=4)), 2) == -3
    assert chunk((qsa._Pool * 1)(_pool(v_bits=4)), 1, D(4, 4, 64, 64)) == -3
    p4 = _pool(v_bits=4)
    assert L.qsa_prompt_attn(1, 16, 0, ctypes.byref(p4), D(4, 4, 64, 64), 1.0, 1, 1, 1 << 30, None) == -3
    assert L.qsa_kv_append((qsa._Pool * 1)(_pool(v_bits=4)), 1, None, D(4, 4, 64, 64), 1, 1, 1, 4, None) == -3


# ------------------------------------------------------------------ the binding's size checks (CPU tensors)
# The C side cannot see the size of a device buffer, so the binding checks every tensor against the sizes the call
# will index it by, before any pointer is taken. CPU tensors suffice: a size error is raised before the device check.
import torch  # noqa: E402


def _cpu_pool(n_kv=2, cap=300, d=128, v_bits=8, index=True):
    g = max(d // 64, 1)
    return qsa.Pool(torch.zeros(n_kv, cap, d, dtype=torch.int8), torch.zeros(n_kv, cap, g),
                    torch.zeros(n_kv, cap, d if v_bits == 8 else d // 2, dtype=torch.int8), torch.zeros(n_kv, cap, g),
                    cap, torch.zeros(n_kv, -(-cap // 64), d) if index else None, v_bits)


SIZE_ERR = r"expected shape|reads or writes|elements|n_valid|index"


def test_binding_rejects_pool_shapes():
    dims = qsa.Dims(12, 2, 128)
    good = _cpu_pool()
    good.check(dims, need_index=True)
    bad_scale = _cpu_pool()
    bad_scale.k_scale = torch.zeros(2, 300, 1)
    bad_v = _cpu_pool()
    bad_v.v = torch.zeros(2, 299, 128, dtype=torch.int8)
    bad_index = _cpu_pool()
    bad_index.index = torch.zeros(2, 4, 128)
    bad_n = _cpu_pool()
    bad_n.n_valid = 301
    for p in (bad_scale, bad_v, bad_index, bad_n):
        with pytest.raises(ValueError, match=SIZE_ERR):
            p.check(dims)
    with pytest.raises(ValueError, match=SIZE_ERR):
        _cpu_pool(index=False).check(dims, need_index=True)
    with pytest.raises(ValueError, match=SIZE_ERR):          # pools for another head count
        good.check(qsa.Dims(12, 3, 128))
    _cpu_pool(v_bits=4).check(dims)                          # K8V4: v holds two codes per byte


def test_binding_rejects_short_buffers():
    dims = qsa.Dims(12, 2, 128)
    p = _cpu_pool()
    q = torch.zeros(3, 12, 128)
    pos = torch.zeros(3, dtype=torch.int32)
    with pytest.raises(ValueError, match=SIZE_ERR):          # pos of 2 rows for 3 rows of q
        qsa.qsa_block_scores(q, pos[:2], p, dims, 5, torch.zeros(3, 2, 5))
    with pytest.raises(ValueError, match=SIZE_ERR):          # score rows narrower than n_blocks
        qsa.qsa_block_scores(q, pos, p, dims, 5, torch.zeros(3, 2, 4))
    with pytest.raises(ValueError, match=SIZE_ERR):          # q with the wrong head count
        qsa.qsa_block_scores(torch.zeros(3, 10, 128), pos, p, dims, 5, torch.zeros(3, 2, 5))
    part = qsa.Partials.empty_like_shape(3, 12, 4, 128, device="cpu")
    ids = torch.zeros(3, 2, 6, dtype=torch.int32)
    with pytest.raises(ValueError, match=SIZE_ERR):          # counts of 2 rows
        qsa.qsa_attn_chunk(q, pos, [p], dims, part, 4, ids=ids, counts=torch.zeros(2, 2, dtype=torch.int32))
    short = qsa.Partials(part.m, part.l, part.o[:2], part.empty)
    with pytest.raises(ValueError, match=SIZE_ERR):          # o of 2 rows of partials
        qsa.qsa_attn_chunk(q, pos, [p], dims, short, 4, blocks_per_chunk=1)
    with pytest.raises(ValueError, match=SIZE_ERR):          # merge output of 2 rows
        qsa.qsa_attn_merge(part, dims, 4, torch.zeros(2, 12, 128))
    with pytest.raises(ValueError, match=SIZE_ERR):
        qsa.qsa_attn_merge(part, dims, 4, torch.zeros(3, 12, 128), lse=torch.zeros(3, 11))
    with pytest.raises(ValueError, match=SIZE_ERR):          # layer ids narrower than k
        qsa.qsa_decode_layer(q, pos, [p], dims, 5, 3, 2, torch.zeros(3, 12, 128), ids=torch.zeros(3, 2, 2))
    with pytest.raises(ValueError, match=SIZE_ERR):
        qsa.qsa_decode_select(q, pos, [p], dims, 5, 3, torch.zeros(3, 2, 3, dtype=torch.int32),
                              torch.zeros(3, dtype=torch.int32))
    with pytest.raises(ValueError, match=SIZE_ERR):          # cells of 1 row for 2 new rows
        qsa.qsa_kv_append([p], dims, torch.zeros(2, 2, 128), torch.zeros(2, 2, 128), torch.zeros(1, dtype=torch.int32))
    with pytest.raises(ValueError, match=SIZE_ERR):          # prompt output of 2 queries for 3
        qsa.qsa_prompt_attn(q, 10, p, dims, torch.zeros(2, 12, 128))
    with pytest.raises(ValueError, match=SIZE_ERR):          # top-k ids narrower than k
        qsa.qsa_topk(torch.zeros(4, 16), 5, torch.zeros(4, 4, dtype=torch.int32), torch.zeros(4, dtype=torch.int32))


def test_noalloc_layer_refuses_oversized_scratch_before_any_hip_call():
    """qsa_decode_layer_noalloc checks its scratch need against the static array's size (QSA_NOALLOC_SCRATCH_BYTES)
    on the host, before touching the device: an oversized layer is refused here, where there is no GPU."""
    L = qsa.lib_handle()
    text = open(HEADER).read()
    assert re.search(r"#define QSA_NOALLOC_SCRATCH_BYTES \(8u << 20\)", text)
    assert qsa.NOALLOC_SCRATCH_BYTES == 8 << 20
    pools = (qsa._Pool * 1)(_pool(cap=200_000, n_valid=65_536))
    need = L.qsa_decode_layer_scratch_bytes(64, GOOD, 1024, 64, 64)
    assert need > qsa.NOALLOC_SCRATCH_BYTES
    st = L.qsa_decode_layer_noalloc(1, 1, 64, pools, 1, None, GOOD, 1024, 64, 64, 1.0, 1, None, None, None, None, None)
    assert st == -4
    # the usual argument checks come first
    assert L.qsa_decode_layer_noalloc(1, 1, 64, pools, 1, None, GOOD, 1024, 64, 0, 1.0, 1, None, None, None, None,
                                      None) == -5
    assert L.qsa_decode_layer_noalloc(1, 1, 64, pools, 1, None, GOOD, 1024, 64, 4, 1.0, None, None, None, None, None,
                                      None) == -1
    assert L.qsa_decode_layer_noalloc(1, 1, 64, pools, 1, None, GOOD, 1024, 64, 4, float("nan"), 1, None, None, None,
                                      None, None) == -5
    assert L.qsa_decode_layer_noalloc(1, 1, 0, pools, 1, None, GOOD, 1024, 64, 4, 1.0, 1, None, None, None, None,
                                      None) == 0
