"""Writes tests/golden/oracle_small_case.json: a small decode + prefill case run
through the CPU reference only (a regression fixture: any later change to the
reference's arithmetic shows up as a diff against it).  Run from the repo root:
    python tests/golden/make_golden.py
"""
import json
import os
import sys

import numpy as np

ROOT = os.path.dirname(os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
sys.path.insert(0, ROOT)

from oracle import oracle as o  # noqa: E402

OUT = os.path.join(os.path.dirname(os.path.abspath(__file__)), "oracle_small_case.json")


def case():
    rng = np.random.default_rng(20261203)
    p = o.Params(num_q_heads=4, num_kv_heads=2, head_dim=16, topk=3, window=256)
    lens = [300, 1100, 40]
    q_lens = [1, 70, 1]
    k = rng.integers(-8, 9, (sum(lens), 2, 16)).astype(np.float32) / 4
    v = rng.integers(-8, 9, (sum(lens), 2, 16)).astype(np.float32) / 4
    q = rng.integers(-8, 9, (sum(q_lens), 4, 16)).astype(np.float32) / 4
    to_bits = lambda x: ((x.astype(np.float32).view(np.uint32) >> 16).astype(np.uint16))
    return p, lens, q_lens, to_bits(q), to_bits(k), to_bits(v)


def run(p, lens, q_lens, q, k, v):
    cu_k = np.concatenate([[0], np.cumsum(lens)]).astype(np.int32)
    cu_q = np.concatenate([[0], np.cumsum(q_lens)]).astype(np.int32)
    return o.forward(p, q, cu_q, k, v, cu_k)


if __name__ == "__main__":
    p, lens, q_lens, q, k, v = case()
    r = run(p, lens, q_lens, q, k, v)
    doc = {
        "_about": "CPU reference outputs for a small varlen case (values k/4, k in [-8, 8]); written by make_golden.py",
        "params": p.__dict__, "lens": lens, "q_lens": q_lens,
        "kc": r["kc"].tolist(), "sel": r["sel"].tolist(), "cnt": r["cnt"].tolist(),
        "scores": [[[[None if not np.isfinite(x) else float(x) for x in row] for row in a] for a in b]
                   for b in r["scores"]],
        "out": r["out"].tolist(), "lse": r["lse"].tolist(),
    }
    with open(OUT, "w") as f:
        json.dump(doc, f)
    print("wrote", OUT)
