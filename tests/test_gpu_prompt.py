"""GPU parity of the whole-prompt sparse prefill (nosa_prefill_sparse): every
query of each prompt attends to the blocks selected for its 64-query block,
chunk by chunk.  Checked against the oracle's forward with the prompt as both
queries and keys; query blocks whose selection sits on a near-tie (relative
gap below the tie band, where fp32 and fp64 may order two blocks differently)
are compared through the stand-alone chain instead.  Different chunk sizes
and the stand-alone chain select the same blocks; their outputs agree within
the rounding of the attention weights (a launch of few workgroups attends each
row group's pages in two halves and combines them, and each half rounds its
weights to bf16 relative to its own running maximum)."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth
from oracle import oracle as ora

from helpers import OUT_MAX_ABS, OUT_MEAN_ABS, gpu_kc_logical, log, make_case
from test_gpu_prefill import check_rows, gpu_prefill, oracle_attend_on_pf

pytestmark = pytest.mark.gpu


def _wl(lens, hq=16, hkv=2, topk=8, window=1024, seed=5, locality=0.0):
    return synth.Workload(lens=list(lens), q_lens=list(lens), num_q_heads=hq, num_kv_heads=hkv,
                          topk=topk, window=window, seed=seed, name="prompt", locality=locality)


def prompt_prefill(c, chunk):
    w = c.w
    B, maxL = w.batch, max(w.lens)
    q = c.inp["q"].cuda()
    cu = synth.cu_from_lens(w.lens, "cuda")
    ws = torch.zeros(nosa.nosa_prefill_sparse_workspace_size(c.p, B, maxL, chunk),
                     dtype=torch.uint8, device="cuda")
    out = torch.full((q.shape[0], w.num_q_heads, 128), float("nan"), device="cuda")
    lse = torch.full((q.shape[0], w.num_q_heads), float("nan"), device="cuda")
    nosa.nosa_prefill_sparse(c.p, c.kv, q, cu, B, maxL, chunk, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def _same(a, b, what):
    """Outputs of two launches of the same attention on the same selection:
    within the output bound, and the log-sum-exp within 1e-4 (fp32 sums)."""
    assert np.isfinite(a[0]).all() and np.isfinite(b[0]).all(), what
    err = np.abs(a[0].astype(np.float64) - b[0])
    assert err.max() <= OUT_MAX_ABS and err.mean() <= OUT_MEAN_ABS / 10, (what, err.max(), err.mean())
    fin = np.isfinite(b[1])
    assert np.array_equal(fin, np.isfinite(a[1])), what
    assert np.abs(a[1][fin] - b[1][fin]).max(initial=0.0) <= 1e-4 * max(1.0, np.abs(b[1][fin]).max(initial=0.0)), what


def _check(c, chunks, tag):
    w = c.w
    c.pg["kc_pool"].fill_(0x7fc0)  # NaN bits: every key the queries use must be rebuilt
    res = {ch: prompt_prefill(c, ch) for ch in chunks}
    cu = synth.cu_from_lens(w.lens).numpy()
    o = ora.forward(c.op, synth.bits(c.inp["q"]), cu, synth.bits(c.inp["k"]),
                    synth.bits(c.inp["v"]), cu)
    for s, L in enumerate(w.lens):
        nc = ora.num_keys(L, c.op)
        if nc:
            assert np.array_equal(gpu_kc_logical(c, s, nc), o["kc"][s, :, :nc]), (tag, s)
    out, lse = res[chunks[0]]
    for ch in chunks[1:]:  # the chunk changes the result only by rounding
        _same(res[ch], (out, lse), (tag, ch))
    g, _ = gpu_prefill(c)  # the stand-alone chain over the same prompt
    _same((g["out"], g["lse"]), (out, lse), tag)
    # every query (near-ties included) against the reference's attention on
    # the chain's selections, which the prompt prefill shares
    oo, ol = oracle_attend_on_pf(c, g["sel"], g["cnt"])
    err = np.abs(out.astype(np.float64) - oo)
    assert err.max() <= OUT_MAX_ABS and err.mean() <= OUT_MEAN_ABS, (tag, "own sets", err.max(),
                                                                      err.mean())
    keep = np.zeros(out.shape[0], bool)
    ex = 0
    for s, L in enumerate(w.lens):
        for r in range(math.ceil(L / 64)):
            e = check_rows(g, o, [(s, r, s, r)], w, f"{tag} s{s} r{r}")
            ex += e
            if e == 0:
                keep[cu[s] + 64 * r:cu[s] + min(64 * r + 64, L)] = True
    err = np.abs(out[keep].astype(np.float64) - o["out"][keep])
    assert np.isfinite(out).all(), tag
    assert err.max() <= OUT_MAX_ABS and err.mean() <= OUT_MEAN_ABS, (tag, err.max(), err.mean())
    fin = np.isfinite(o["lse"][keep])
    assert np.array_equal(fin, np.isfinite(lse[keep])), tag
    lerr = np.abs(lse[keep][fin].astype(np.float64) - o["lse"][keep][fin])
    assert lerr.max() <= 1e-3 * max(1.0, np.abs(o["lse"][keep][fin]).max()), tag
    log(f"{tag}: ok ({keep.sum()} of {keep.size} queries against the oracle, "
        f"tie exemptions {ex})")


@pytest.mark.parametrize("lens,chunks", [
    ([3000, 1281, 64, 700], [512, 64, 4096]),
    ([40], [64]),
    ([1], [64, 128]),
    ([4100, 33], [1024, 192])])
def test_prompt_prefill_lengths(lens, chunks):
    log(f"case: prompt prefill lens {lens} chunks {chunks}")
    c = make_case(_wl(lens, seed=sum(lens) % 97))
    _check(c, chunks, f"prompt {lens}")


@pytest.mark.parametrize("hq,hkv,topk,locality", [(32, 8, 6, 0.0), (12, 3, 4, 0.5),
                                                   (16, 2, 0, 0.0), (8, 8, 1000, 0.0)])
def test_prompt_prefill_heads_and_budget(hq, hkv, topk, locality):
    log(f"case: prompt prefill heads {hq}/{hkv} topk {topk} locality {locality}")
    c = make_case(_wl([1900, 700], hq=hq, hkv=hkv, topk=topk, seed=hq + topk, locality=locality))
    _check(c, [512, 256], f"prompt {hq}/{hkv} k{topk} loc{locality}")


def test_prompt_prefill_errors():
    c = make_case(_wl([300]))
    ws = torch.zeros(1 << 20, dtype=torch.uint8, device="cuda")
    for bad in (0, 100, -64):
        with pytest.raises(nosa.NosaError) as e:
            nosa.nosa_prefill_sparse_workspace_size(c.p, 1, 300, bad)
        assert e.value.status == 2
    out = torch.empty(300, 16, 128, device="cuda")
    with pytest.raises(nosa.NosaError) as e:
        nosa.nosa_prefill_sparse(c.p, c.kv, c.inp["q"].cuda(), synth.cu_from_lens([300], "cuda"),
                                 1, 300, 64, out, None, ws[:100])
    assert e.value.status == 4
