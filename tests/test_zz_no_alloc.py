"""nosa_decode_step_static (the decode step for callers that cannot allocate:
its partials live in a static device array of the library) against
nosa_decode_step with a caller's workspace: two calls in a row, the second on
a smaller batch, each bitwise identical to the workspace entry point on the
same inputs (same kernels and launch plan) and within the output bound of the
reference on the step's own selection; then the static call captured in a
HIP graph and replayed, with other work between replays, every replay equal
to the eager result."""
import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth

from helpers import (build_kc, compare_outputs, compare_selection, cu_dev, live_lens, log,
                     make_case, oracle_attend_on, oracle_step, workspace)

pytestmark = pytest.mark.gpu


def _wl(lens, topk, seed, hq=16, hkv=2):
    return synth.Workload(lens=list(lens), num_q_heads=hq, num_kv_heads=hkv, topk=topk,
                          planted=2, seed=seed, name="static")


def _bufs(c):
    W = c.w
    max_sel = W.topk + W.window // W.block_size
    max_nb = (max(live_lens(c, 0)) + 63) // 64
    return dict(out=torch.full((c.B, W.num_q_heads, 128), float("nan"), device="cuda"),
                lse=torch.full((c.B, W.num_q_heads), float("nan"), device="cuda"),
                sel=torch.full((c.B, 1, W.num_kv_heads, max_sel), -7, dtype=torch.int32,
                               device="cuda"),
                cnt=torch.full((c.B, 1, W.num_kv_heads), -7, dtype=torch.int32, device="cuda"),
                scores=torch.full((c.B, 1, W.num_kv_heads, max_nb), float("nan"),
                                  device="cuda"))


def _run(c, static):
    lens = live_lens(c, 0)
    b = _bufs(c)
    q, cu, maxL = c.inp["q"].cuda(), cu_dev(lens), max(lens)
    if static:
        nosa.nosa_decode_step_static(c.p, c.kv, q, cu, c.B, maxL, b["out"], b["lse"],
                                     sel_idx=b["sel"], sel_count=b["cnt"],
                                     block_scores=b["scores"])
    else:
        nosa.nosa_decode_step(c.p, c.kv, q, cu, c.B, maxL, b["out"], b["lse"], workspace(c, maxL),
                              sel_idx=b["sel"], sel_count=b["cnt"], block_scores=b["scores"])
    return b


def _host(b):
    torch.cuda.synchronize()
    return {k: v.cpu().numpy() for k, v in b.items()}


def test_static_scratch_matches_workspace_entry_point():
    big = make_case(_wl([40000, 9000, 3000, 17000], topk=64, seed=41, hq=32, hkv=8))
    small = make_case(_wl([2500, 700], topk=8, seed=42))
    assert nosa.nosa_workspace_size(big.p, big.B, 1, 40000) <= nosa.STATIC_SCRATCH_BYTES
    refs = []
    for c in (big, small):
        build_kc(c, [L - 1 for L in live_lens(c, 0)])
        refs.append(_host(_run(c, static=False)))
    # two static calls in a row, the second on the smaller batch (the key each
    # step appends is the one already there, so the inputs are unchanged)
    got = [_run(big, static=True), _run(small, static=True)]
    got = [_host(g) for g in got]
    for c, r, g, tag in ((big, refs[0], got[0], "big"), (small, refs[1], got[1], "small")):
        for k in ("out", "lse", "sel", "cnt", "scores"):
            assert np.array_equal(g[k], r[k], equal_nan=True), (tag, k)
        lens = live_lens(c, 0)
        o = oracle_step(c, 0)
        ex = compare_selection(g["sel"], g["cnt"], o["sel"], o["cnt"], o["scores"], lens, c.w)
        oo, ol = oracle_attend_on(c, 0, g["sel"], g["cnt"])
        compare_outputs(g["out"], g["lse"], oo, ol, f"static {tag} (own set)")
        if ex == 0:
            compare_outputs(g["out"], g["lse"], o["out"], o["lse"], f"static {tag}")
        log(f"static scratch, {tag} batch: ok (tie exemptions {ex})")


def test_static_scratch_graph_replays():
    c = make_case(_wl([6000, 1200], topk=16, seed=43))
    lens = live_lens(c, 0)
    build_kc(c, [L - 1 for L in lens])
    eager = _host(_run(c, static=True))
    b = _bufs(c)
    q, cu = c.inp["q"].cuda(), cu_dev(lens)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        nosa.nosa_decode_step_static(c.p, c.kv, q, cu, c.B, max(lens), b["out"], b["lse"],
                                     sel_idx=b["sel"], sel_count=b["cnt"],
                                     block_scores=b["scores"])
    other = make_case(_wl([3000], topk=4, seed=44))
    build_kc(other, [L - 1 for L in live_lens(other, 0)])
    for rep in range(3):
        for t in b.values():
            t.fill_(-1)
        graph.replay()
        got = _host(b)
        for k in eager:
            assert np.array_equal(got[k], eager[k], equal_nan=True), (rep, k)
        _host(_run(other, static=True))  # eager work on the same scratch between replays
    log("static scratch: 3 graph replays equal the eager step")
