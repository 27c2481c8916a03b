"""Writes tests/golden/tiny_decode_oracle.json from the FP64 oracle alone (no GPU code is imported).

Run from the repository root: python tests/golden/make_golden.py
The fixture freezes the oracle's ids and a few output values for the 1-query, 4/1-head, 1,024-cell decode
workload (top-8 of 16 blocks), so an accidental change to the oracle's arithmetic shows up as a failed test.
"""
import json
import os
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

import numpy as np  # noqa: E402

import oracle  # noqa: E402
import synth  # noqa: E402


def main():
    w = synth.workload("tiny_decode")
    pool = w.pools[0]
    nb = -(-pool.n_valid // oracle.BLOCK)
    r = oracle.block_index(pool)
    s = oracle.block_scores(w.q, w.pos, r, w.n_kv_heads, pool.n_valid, nb)
    ids, counts = oracle.topk(s.reshape(-1, nb), w.topk)
    out, lse = oracle.attn(w.q, w.pos, pool, w.n_kv_heads, ids=ids.reshape(1, 1, -1), counts=counts.reshape(1, 1))
    fixture = {
        "workload": "tiny_decode (seed 1000)",
        "source": "FP64 oracle, tests/golden/make_golden.py",
        "scores": [float(x) for x in s[0, 0]],
        "ids": [int(x) for x in ids[0]],
        "count": int(counts[0]),
        "out_head0_first8": [float(x) for x in out[0, 0, :8]],
        "out_head3_last8": [float(x) for x in out[0, 3, -8:]],
        "lse": [float(x) for x in lse[0]],
    }
    path = os.path.join(os.path.dirname(os.path.abspath(__file__)), "tiny_decode_oracle.json")
    with open(path, "w") as f:
        json.dump(fixture, f, indent=1)
        f.write("\n")


if __name__ == "__main__":
    main()
