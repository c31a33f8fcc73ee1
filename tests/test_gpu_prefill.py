"""GPU parity of the chunked sparse prefill (cu_seqlens_q given): block
importance per 64-query block, selection, causal attention on MFMA.  The
131072-token workload is checked on sampled query blocks: the CPU reference
solves each sampled block as its own problem with the context cut after the
block's last query, which is the same computation (nothing later is visible)."""
import math

import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth
from oracle import oracle as ora

from helpers import (OUT_MAX_ABS, OUT_MEAN_ABS, TIE_BAND, DecodeCase, build_kc, local_blocks, log,
                     make_case)

pytestmark = pytest.mark.gpu


def _wl(lens, q_lens, hq=16, hkv=2, topk=8, window=1024, seed=3, locality=0.0):
    return synth.Workload(lens=list(lens), q_lens=list(q_lens), num_q_heads=hq, num_kv_heads=hkv,
                          topk=topk, window=window, seed=seed, name="pf", locality=locality)


def gpu_prefill(c):
    w = c.w
    B = w.batch
    maxL, maxLq = max(w.lens), max(w.q_lens)
    max_qblk = max(1, math.ceil(maxLq / 64))
    max_nb = math.ceil(maxL / 64)
    max_sel = w.topk + w.window // 64
    q = c.inp["q"].cuda()
    cu_q = c.inp["cu_q"].cuda().to(torch.int32)
    cu_k = synth.cu_from_lens(w.lens, "cuda")
    scores = torch.full((B, max_qblk, w.num_kv_heads, max_nb), float("nan"), device="cuda")
    ws = torch.zeros(nosa.nosa_workspace_size(c.p, B, maxLq, maxL), dtype=torch.uint8,
                     device="cuda")
    nosa.nosa_block_scores(c.p, c.kv, q, cu_q, cu_k, B, maxLq, maxL, scores, ws)
    sel = torch.full((B, max_qblk, w.num_kv_heads, max_sel), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, max_qblk, w.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    nosa.nosa_select_blocks(c.p, scores, cu_q, cu_k, B, maxLq, maxL, sel, cnt)
    out = torch.full((q.shape[0], w.num_q_heads, 128), float("nan"), device="cuda")
    lse = torch.full((q.shape[0], w.num_q_heads), float("nan"), device="cuda")
    nosa.nosa_sparse_attend(c.p, c.kv, q, cu_q, cu_k, B, maxLq, maxL, sel, cnt, out, lse, ws)
    torch.cuda.synchronize()
    res = dict(scores=scores.cpu().numpy(), sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(),
               out=out.cpu().numpy(), lse=lse.cpu().numpy())
    return res, (q, cu_q, cu_k, out, lse, ws)


def attend_with(c, sel_np, cnt_np, args):
    q, cu_q, cu_k, out, lse, ws = args
    w = c.w
    sel = torch.as_tensor(np.ascontiguousarray(sel_np), dtype=torch.int32).cuda()
    cnt = torch.as_tensor(np.ascontiguousarray(cnt_np), dtype=torch.int32).cuda()
    out.fill_(float("nan"))
    lse.fill_(float("nan"))
    nosa.nosa_sparse_attend(c.p, c.kv, q, cu_q, cu_k, w.batch, max(w.q_lens), max(w.lens), sel,
                            cnt, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_attend_on_pf(c, sel, cnt):
    """The reference's attention for every query of the case over the given
    per-q-block selections [B][max_qblk][Hkv][>= max_sel]."""
    w = c.w
    max_sel = w.topk + w.window // 64
    return ora.sparse_attend(c.op, synth.bits(c.inp["q"]), c.inp["cu_q"].cpu().numpy(),
                             synth.bits(c.inp["k"]), synth.bits(c.inp["v"]),
                             synth.cu_from_lens(w.lens).numpy(),
                             np.ascontiguousarray(sel[..., :max_sel]), cnt)


def qblock_nb(L, Lq, r):
    p_last = L - Lq + min(64 * r + 64, Lq) - 1
    return p_last // 64 + 1


def check_rows(g, o, rows, w, tag):
    """rows: list of (s, r, s_o, r_o): GPU row (s, r) against reference row (s_o, r_o)."""
    k_loc = local_blocks(w)  # forced like the window
    wb = w.window // 64 + k_loc
    exempt = 0
    for (s, r, so, ro) in rows:
        L, Lq = w.lens[s], w.q_lens[s]
        nb = qblock_nb(L, Lq, r)
        for gi in range(w.num_kv_heads):
            gs = g["scores"][s, r, gi, :nb].astype(np.float64)
            os_ = o["scores"][so, ro, gi, :nb]
            fin = np.isfinite(os_)
            assert np.array_equal(fin, np.isfinite(gs)), (tag, s, r, gi)
            if fin.any():
                floor = 1e-6 * np.abs(os_[fin]).max()
                rel = np.abs(gs[fin] - os_[fin]) / (np.abs(os_[fin]) + floor)
                assert rel.max() <= TIE_BAND, (tag, s, r, gi, rel.max())
            n = int(o["cnt"][so, ro, gi])
            assert int(g["cnt"][s, r, gi]) == n, (tag, s, r, gi)
            a = g["sel"][s, r, gi, :n].tolist()
            b = o["sel"][so, ro, gi, :n].tolist()
            if a != b:
                ncand = max(nb - wb, 0)
                sc = os_[:ncand]
                k = min(w.topk - k_loc, ncand)
                order = sorted(range(ncand), key=lambda x: (-sc[x], x))
                kth = sc[order[k - 1]]
                nxt = sc[order[k]] if k < ncand else -np.inf
                assert abs(kth - nxt) / max(abs(kth), abs(nxt)) < TIE_BAND, (tag, s, r, gi)
                for x in set(a) ^ set(b):
                    assert abs(sc[x] - kth) <= TIE_BAND * abs(kth), (tag, s, r, gi, x)
                exempt += 1
    return exempt


def compare_out(gout, glse, oout, olse, tag):
    err = np.abs(gout.astype(np.float64) - oout)
    assert np.isfinite(gout).all(), tag
    assert err.max() <= OUT_MAX_ABS and err.mean() <= OUT_MEAN_ABS, (tag, err.max(), err.mean())
    lerr = np.abs(glse.astype(np.float64) - olse)
    fin = np.isfinite(olse)
    assert np.array_equal(fin, np.isfinite(glse)), tag
    assert (lerr[fin].max() if fin.any() else 0) <= 1e-3 * max(1.0, np.abs(olse[fin]).max()), tag


def _full(c, tag):
    w = c.w
    build_kc(c, w.lens)
    g, args = gpu_prefill(c)
    o = ora.forward(c.op, synth.bits(c.inp["q"]), c.inp["cu_q"].cpu().numpy(), synth.bits(c.inp["k"]),
                    synth.bits(c.inp["v"]), synth.cu_from_lens(w.lens).numpy())
    rows = [(s, r, s, r) for s in range(w.batch) for r in range(math.ceil(w.q_lens[s] / 64))]
    ex = check_rows(g, o, rows, w, tag)
    out, lse = attend_with(c, o["sel"], o["cnt"], args)
    compare_out(out, lse, o["out"], o["lse"], tag + " attend(oracle sets)")
    # the chain's output against the reference's attention on the chain's own
    # sets (always), and against the reference's output when the sets agree
    oo, ol = oracle_attend_on_pf(c, g["sel"], g["cnt"])
    compare_out(g["out"], g["lse"], oo, ol, tag + " chain (own sets)")
    if ex == 0:
        compare_out(g["out"], g["lse"], o["out"], o["lse"], tag + " chain")
    log(f"{tag}: ok (tie exemptions {ex})")


@pytest.mark.parametrize("hq,hkv", [(16, 2), (32, 8), (16, 1), (12, 3), (8, 8)])
def test_prefill_head_groups(hq, hkv):
    log(f"case: prefill heads {hq}/{hkv}")
    c = make_case(_wl([3000], [200], hq=hq, hkv=hkv, seed=hq + hkv))
    _full(c, f"pf{hq}/{hkv}")


@pytest.mark.parametrize("lens,q_lens", [
    ([700], [150]), ([1280], [128]), ([1281], [1]), ([2000, 1100, 64], [64, 300, 64]),
    ([3333, 40], [333, 40]), ([5000], [5000])])
def test_prefill_lengths(lens, q_lens):
    log(f"case: prefill lens {lens} q {q_lens}")
    c = make_case(_wl(lens, q_lens, seed=sum(lens) + sum(q_lens)))
    _full(c, f"pf{lens}/{q_lens}")


@pytest.mark.parametrize("topk", [0, 3, 1000])
def test_prefill_topk(topk):
    log(f"case: prefill topk {topk}")
    c = make_case(_wl([4000], [260], topk=topk, seed=topk + 7))
    _full(c, f"pf topk {topk}")


@pytest.mark.parametrize("locality", [0.5, 0.75])
def test_prefill_locality(locality):
    log(f"case: prefill locality {locality}")
    c = make_case(_wl([6000, 2200], [400, 130], topk=12, seed=int(locality * 8), locality=locality))
    _full(c, f"pf loc {locality}")


def test_prefill_logits_far_below_the_span_start():
    """Logits spread far beyond the float range of exp2: every query and,
    negated, the keys of tokens 0 .. 527 share a direction u (entries +-1) at
    3.5 times the noise, so pooled keys 0 .. 31 -- the first pair of key
    tiles of the first span -- score 180 or more (log2 units) below the
    span's later keys for every row.  The scoring pass's reference taken from
    that pair overflows on the later keys and the span is redone with the
    maximum tracked.  The blocks that compete for the top-k keep ordinary
    scores (the pushed-down ones only lose), so everything must match the
    reference."""
    log("case: prefill with logits far below the span start")
    w = _wl([3000], [200], seed=41)
    inp = synth.make_inputs(w)
    gen = torch.Generator().manual_seed(41)
    u = torch.randint(0, 2, (w.head_dim,), generator=gen).float() * 2 - 1
    inp["q"] = (inp["q"].float() + 3.5 * u).to(torch.bfloat16)
    k = inp["k"].float()
    k[0:528] -= 3.5 * u
    inp["k"] = k.to(torch.bfloat16)
    pg = synth.to_paged(inp, w, permute=True, device="cuda")
    p = nosa.params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    op = ora.Params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    kv = nosa.paged_kv(pg["k_pool"], pg["v_pool"], pg["kc_pool"], pg["block_table"])
    c = DecodeCase(w, inp, pg, p, op, kv)
    _full(c, "pf far below")


def test_prefill_131072_sampled_query_blocks():
    """The 2048-query chunk at the end of a 131072-token context, eight of its
    32 query blocks (first, last and six between) against the reference,
    which solves each as its own problem cut after the block's last query.
    For every sampled block: importance and selection (near-tie band), the
    chain's output against the reference's attention on the chain's own
    selection, the stand-alone attention on the reference's selection against
    the reference's output, and the chain's output against it directly when
    the selections agree.  Every sampled block is compared."""
    log("case: prefill-2048-of-131072, sampled query blocks")
    w = synth.config(5)
    c = make_case(w, gen_device="cuda")
    build_kc(c, w.lens)
    g, args = gpu_prefill(c)
    L, Lq = w.lens[0], w.q_lens[0]
    assert np.isfinite(g["out"]).all()
    sampled = (0, 4, 9, 13, 18, 22, 27, 31)
    sel_o = g["sel"].copy()
    cnt_o = g["cnt"].copy()
    refs = {}
    ex = 0
    for r in sampled:
        p_last = L - Lq + 64 * r + 63
        k = synth.bits(c.inp["k"][:p_last + 1])
        v = synth.bits(c.inp["v"][:p_last + 1])
        q = synth.bits(c.inp["q"][64 * r:64 * r + 64])
        cu_q, cu_k = np.array([0, 64], np.int32), np.array([0, p_last + 1], np.int32)
        o = ora.forward(c.op, q, cu_q, k, v, cu_k)
        e = check_rows(g, o, [(0, r, 0, 0)], w, f"c5 r{r}")
        ex += e
        rows = slice(64 * r, 64 * r + 64)
        oo, ol = ora.sparse_attend(c.op, q, cu_q, k, v, cu_k, g["sel"][:, r:r + 1], g["cnt"][:, r:r + 1])
        compare_out(g["out"][rows], g["lse"][rows], oo, ol, f"c5 r{r} chain (own set)")
        if e == 0:
            compare_out(g["out"][rows], g["lse"][rows], o["out"], o["lse"], f"c5 r{r} chain")
        sel_o[0, r] = o["sel"][0, 0]
        cnt_o[0, r] = o["cnt"][0, 0]
        refs[r] = o
        log(f"c5 q-block {r}: chain ok (exemptions {e})")
    out, lse = attend_with(c, sel_o, cnt_o, args)
    for r in sampled:
        rows = slice(64 * r, 64 * r + 64)
        compare_out(out[rows], lse[rows], refs[r]["out"], refs[r]["lse"], f"c5 r{r} attend(oracle set)")
    log(f"c5: {len(sampled)} of 32 query blocks compared, tie exemptions {ex}")
