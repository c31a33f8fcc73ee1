"""GPU parity at the full sizes of the decode workloads, in the launch
configuration the benchmark times (one nosa_decode_step call per step on the
whole batch).  Inputs are generated on the GPU from the seeded generator; the
CPU reference sees host copies of the same inputs, for every sequence where it
is fast enough and for sampled sequences of the 64K batch."""
import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import synth
from oracle import oracle as ora

from helpers import (build_kc, compare_outputs, compare_scores, compare_selection, gpu_attend,
                     gpu_decode_step, gpu_kc_logical, live_lens, log, make_case, oracle_step)

pytestmark = pytest.mark.gpu


def _check_step(c, step, seqs=None, tag=""):
    g = gpu_decode_step(c, step)
    o = oracle_step(c, step, seqs=seqs)
    lens = live_lens(c, step)
    rows = list(range(c.B)) if seqs is None else list(seqs)
    sub = {k: g[k][rows] for k in ("sel", "cnt", "scores", "out", "lse")}
    lens_s = [lens[s] for s in rows]
    compare_scores(sub["scores"], o["scores"], lens_s, c.w)
    ex = compare_selection(sub["sel"], sub["cnt"], o["sel"], o["cnt"], o["scores"], lens_s, c.w)
    if ex == 0:
        compare_outputs(sub["out"], sub["lse"], o["out"], o["lse"], tag + " fused")
    # attention on the reference's own selection through the stand-alone entry
    if seqs is None:
        out, lse = gpu_attend(c, step, o["sel"], o["cnt"])
        compare_outputs(out, lse, o["out"], o["lse"], tag + " attend")
    log(f"{tag}: step {step} ok (tie exemptions {ex})")
    return g, o


def test_decode_b8_16k_all_steps():
    """256 consecutive decode steps with appends; full comparison at the
    window-shift steps and at the first and last one; the pooled keys after
    the last append equal the reference's."""
    log("case: decode-b8-16k, 256 steps")
    w = synth.config(2)
    c = make_case(w, gen_device="cuda")
    build_kc(c, [L - 1 for L in w.lens])
    check = {0, 1, 63, 64, 127, 128, 191, 255}
    for step in range(256):
        if step in check:
            _check_step(c, step, tag="c2")
        else:
            gpu_decode_step(c, step)
    lens = live_lens(c, 255)
    k, _, cu = synth.packed_live(c.inp, w, 255)
    o = ora.compress_keys(c.op, synth.bits(k), cu.numpy())
    for s in range(w.batch):
        nc = ora.num_keys(lens[s], c.op)
        assert np.array_equal(gpu_kc_logical(c, s, nc), o[s, :, :nc]), s
    # the planted blocks are found at every checked step
    g = gpu_decode_step(c, 255)
    for s in range(w.batch):
        for gi in range(w.num_kv_heads):
            chosen = set(g["sel"][s, 0, gi, :g["cnt"][s, 0, gi]].tolist())
            assert set(c.inp["planted"][s * w.num_kv_heads + gi]) <= chosen


def test_decode_varlen_b32_permuted_pages():
    log("case: decode-varlen-b32")
    w = synth.config(3)
    c = make_case(w, gen_device="cuda")
    build_kc(c, [L - 1 for L in w.lens])
    _check_step(c, 0, tag="c3")


def test_decode_b16_64k_gqa4_sampled():
    log("case: decode-b16-64k, sequences 0 and 15 against the reference")
    w = synth.config(4)
    c = make_case(w, gen_device="cuda")
    build_kc(c, [L - 1 for L in w.lens])
    g, _ = _check_step(c, 0, seqs=[0, 15], tag="c4")
    # every sequence: sizes, ordering and window of the selection are valid
    for s in range(w.batch):
        nb = (w.lens[s] + 63) // 64
        for gi in range(w.num_kv_heads):
            n = g["cnt"][s, 0, gi]
            sel = g["sel"][s, 0, gi, :n]
            assert n == min(nb, w.topk + 16)
            assert np.all(np.diff(sel) > 0) and sel[-1] == nb - 1
            assert set(range(nb - 16, nb)) <= set(sel.tolist())
            assert set(c.inp["planted"][s * w.num_kv_heads + gi]) <= set(sel.tolist())
    assert np.isfinite(g["out"]).all() and np.isfinite(g["lse"]).all()
    torch.cuda.empty_cache()
