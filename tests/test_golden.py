"""Golden fixtures: the pages' printed sparse configuration, and a regression
fixture of the CPU reference (written by tests/golden/make_golden.py)."""
import json
import os

import numpy as np

from oracle.oracle import Params
from block_sparse_attention_nosa_amd import synth

HERE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def test_default_parameters_match_the_printed_table():
    g = json.load(open(os.path.join(HERE, "nosa1b_sparse_config.json")))
    p = Params()
    assert (p.topk, p.window, p.block_size, p.kernel, p.stride) == (
        g["topk_blocks"], g["window_tokens"], g["block_size"], g["pool_kernel"], g["pool_stride"])
    assert (p.num_q_heads, p.num_kv_heads) == (g["num_q_heads"], g["num_kv_heads"])
    assert p.head_dim == g["hidden_size"] // g["num_q_heads"]
    assert p.window // p.block_size == 16          # "about 16 nearby blocks"
    # the 8B-scale workload's budget: 96 blocks of 64 tokens = 6144 tokens
    w4 = synth.config(4)
    assert w4.topk * w4.block_size == g["budget_tokens_example"]
    assert g["budget_tokens_example"] / g["budget_context_tokens"] == g["budget_sparsity"]
    w2 = synth.config(2)
    assert (w2.topk, w2.window, w2.num_q_heads, w2.num_kv_heads) == (64, 1024, 16, 2)


def test_oracle_regression_fixture(oracle):
    import importlib.util
    spec = importlib.util.spec_from_file_location("make_golden", os.path.join(HERE, "make_golden.py"))
    mg = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mg)
    g = json.load(open(os.path.join(HERE, "oracle_small_case.json")))
    p, lens, q_lens, q, k, v = mg.case()
    # the fixture predates the locality field; it was written with plain top-k
    assert g["lens"] == lens and g["q_lens"] == q_lens and p.locality == 0.0
    assert g["params"] == {key: p.__dict__[key] for key in g["params"]}
    r = mg.run(p, lens, q_lens, q, k, v)
    assert np.array_equal(r["kc"], np.array(g["kc"], dtype=np.uint16))
    assert np.array_equal(r["sel"], np.array(g["sel"]))
    assert np.array_equal(r["cnt"], np.array(g["cnt"]))
    sc = np.array([[[[np.nan if x is None else x for x in row] for row in a] for a in b]
                   for b in g["scores"]])
    fin = np.isfinite(sc)
    assert np.array_equal(fin, np.isfinite(r["scores"]))
    np.testing.assert_allclose(r["scores"][fin], sc[fin], rtol=1e-13)
    np.testing.assert_allclose(r["out"], np.array(g["out"]), rtol=0, atol=1e-13)
    np.testing.assert_allclose(r["lse"], np.array(g["lse"]), rtol=0, atol=1e-13)
