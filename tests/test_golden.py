"""Golden fixtures for the oracle (CPU only): hand-derived closed forms and a frozen oracle regression."""
import json
import os

import numpy as np

import oracle
import synth

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _pool(k0, v0, cap=64):
    n = len(k0)
    k = np.zeros((1, cap, 64), np.int8)
    v = np.zeros((1, cap, 64), np.int8)
    k[0, :n, 0] = k0
    v[0, :n, 0] = v0
    ks = np.ones((1, cap, 1), np.float32)
    vs = np.ones((1, cap, 1), np.float32)
    return synth.Pool(k, ks, v, vs, cap, n)


def test_closed_forms():
    with open(os.path.join(GOLDEN, "closed_forms.json")) as f:
        cases = json.load(f)["cases"]
    for c in cases:
        pool = _pool(c["k0"], c["v0"])
        q = np.zeros((1, 1, 64), np.float32)
        q[0, 0, 0] = c["q0"]
        out, lse = oracle.attn(q, np.array([c["pos"]], np.int32), pool, 1, sm_scale=c["sm_scale"])
        assert abs(out[0, 0, 0] - c["out0"]) < 1e-13, c["name"]
        assert np.all(out[0, 0, 1:] == 0)
        assert abs(lse[0, 0] - c["lse"]) < 1e-13, c["name"]


def test_oracle_regression_fixture():
    with open(os.path.join(GOLDEN, "tiny_decode_oracle.json")) as f:
        g = json.load(f)
    w = synth.workload("tiny_decode")
    pool = w.pools[0]
    nb = -(-pool.n_valid // oracle.BLOCK)
    s = oracle.block_scores(w.q, w.pos, oracle.block_index(pool), 1, pool.n_valid, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), w.topk)
    out, lse = oracle.attn(w.q, w.pos, pool, 1, ids=ids.reshape(1, 1, -1), counts=counts.reshape(1, 1))
    np.testing.assert_allclose(s[0, 0], g["scores"], rtol=0, atol=1e-15)
    assert list(ids[0]) == g["ids"] and counts[0] == g["count"]
    np.testing.assert_allclose(out[0, 0, :8], g["out_head0_first8"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(out[0, 3, -8:], g["out_head3_last8"], rtol=0, atol=1e-15)
    np.testing.assert_allclose(lse[0], g["lse"], rtol=0, atol=1e-14)
