"""Shared pieces of the GPU parity tests: build a decode case from the seeded
generator, run the HIP path through the C ABI and the CPU reference on the same
inputs, and compare them under the stated rules:
  * pooled keys: bit-exact;
  * block importance: relative error <= 1e-4 (fp32 vs fp64);
  * selections: identical, except where the reference's k-th and (k+1)-th
    candidate scores differ by < 1e-4 relative; then every block the two sets
    disagree on must lie inside that band;
  * attention output: max-abs <= 1e-2 and mean-abs <= 1e-3 (bf16 inputs, fp32
    accumulation), compared on the reference's own selection.
"""
from __future__ import annotations

import sys
from dataclasses import dataclass

import math

import numpy as np
import torch

from block_sparse_attention_nosa_amd import nosa, synth
from oracle import oracle as ora

TIE_BAND = 1e-4
OUT_MAX_ABS = 1e-2
OUT_MEAN_ABS = 1e-3


def log(msg: str):
    print(msg, flush=True)
    sys.stdout.flush()


@dataclass
class DecodeCase:
    w: synth.Workload
    inp: dict
    pg: dict
    p: nosa.nosa_params
    op: ora.Params
    kv: nosa.nosa_paged_kv

    @property
    def B(self):
        return self.w.batch


def make_case(w: synth.Workload, gen_device="cpu", permute=True) -> DecodeCase:
    inp = synth.make_inputs(w, device=gen_device)
    pg = synth.to_paged(inp, w, permute=permute, device="cuda")
    p = nosa.params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    op = ora.Params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    kv = nosa.paged_kv(pg["k_pool"], pg["v_pool"], pg["kc_pool"], pg["block_table"])
    return DecodeCase(w, inp, pg, p, op, kv)


def live_lens(c: DecodeCase, step: int):
    return [L + step for L in c.w.lens]


def cu_dev(lens):
    return synth.cu_from_lens(lens, "cuda")


def build_kc(c: DecodeCase, lens, valid=None):
    """Pooled keys for the first `lens` tokens (full build, or from `valid`)."""
    cu = cu_dev(lens)
    vl = None if valid is None else torch.tensor(valid, dtype=torch.int32, device="cuda")
    nosa.nosa_compress_keys(c.p, c.kv, cu, vl, c.B, max(lens))


def gpu_kc_logical(c: DecodeCase, s: int, nc: int) -> np.ndarray:
    """GPU pooled keys of sequence s in logical order: [Hkv][nc][d] bf16 bits."""
    slots = c.w.block_size // c.w.stride
    d = c.w.head_dim
    table = c.pg["block_table"][s].cpu()
    j = torch.arange(nc)
    pages = table[(j // slots)].long()
    # stored page -> logical [slot][channel]
    idx = synth.page_index("kc", c.w.block_size, d, c.w.stride)
    stored = c.pg["kc_pool"].cpu()
    logical = torch.empty_like(stored)
    logical[:, :, idx] = stored
    kc = logical.view(stored.shape[0], stored.shape[1], slots, d)[pages, :, (j % slots)]  # [nc, Hkv, d]
    return synth.bits(kc.permute(1, 0, 2))


def workspace(c: DecodeCase, max_seqlen_k: int) -> torch.Tensor:
    n = nosa.nosa_workspace_size(c.p, c.B, 1, max_seqlen_k)
    return torch.zeros(n, dtype=torch.uint8, device="cuda")


def gpu_decode_step(c: DecodeCase, step: int = 0):
    """Run one fused decode step at live length lens+step.  Kc must be valid
    for lens+step-1 tokens."""
    lens = live_lens(c, step)
    maxL = max(lens)
    W = c.w
    max_nb = (maxL + W.block_size - 1) // W.block_size
    max_sel = W.topk + W.window // W.block_size
    out = torch.full((c.B, W.num_q_heads, W.head_dim), float("nan"), device="cuda")
    lse = torch.full((c.B, W.num_q_heads), float("nan"), device="cuda")
    # (at least one column: an empty tensor has no address, and the list is
    # passed whenever the counts are)
    sel_buf = torch.full((c.B, 1, W.num_kv_heads, max(max_sel, 1)), -7, dtype=torch.int32, device="cuda")
    sel = sel_buf if max_sel > 0 else sel_buf[..., :0]
    cnt = torch.full((c.B, 1, W.num_kv_heads), -7, dtype=torch.int32, device="cuda")
    scores = torch.full((c.B, 1, W.num_kv_heads, max_nb), float("nan"), device="cuda")
    ws = workspace(c, maxL)
    nosa.nosa_decode_step(c.p, c.kv, c.inp["q"].to("cuda"), cu_dev(lens), c.B, maxL, out, lse,
                          ws, sel_idx=sel_buf, sel_count=cnt, block_scores=scores)
    torch.cuda.synchronize()
    return dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), sel=sel.cpu().numpy(),
                cnt=cnt.cpu().numpy(), scores=scores.cpu().numpy())


def gpu_attend(c: DecodeCase, step: int, sel: np.ndarray, cnt: np.ndarray):
    lens = live_lens(c, step)
    maxL = max(lens)
    W = c.w
    out = torch.full((c.B, W.num_q_heads, W.head_dim), float("nan"), device="cuda")
    lse = torch.full((c.B, W.num_q_heads), float("nan"), device="cuda")
    ws = workspace(c, maxL)
    sel_d = torch.as_tensor(np.ascontiguousarray(sel), dtype=torch.int32).cuda()
    cnt_d = torch.as_tensor(np.ascontiguousarray(cnt), dtype=torch.int32).cuda()
    nosa.nosa_sparse_attend(c.p, c.kv, c.inp["q"].to("cuda"), None, cu_dev(lens), c.B, 1, maxL,
                            sel_d, cnt_d, out, lse, ws)
    torch.cuda.synchronize()
    return out.cpu().numpy(), lse.cpu().numpy()


def oracle_inputs(c: DecodeCase, step: int = 0, seqs=None):
    """Host bit patterns (q, k, v) and cu_seqlens_k of the live tokens at
    `step`, for every sequence or for the listed ones."""
    k, v, cu = synth.packed_live(c.inp, c.w, step)
    q = c.inp["q"]
    if seqs is not None:
        ks, vs, lens = [], [], []
        cu_np = cu.numpy()
        for s in seqs:
            ks.append(k[cu_np[s]:cu_np[s + 1]])
            vs.append(v[cu_np[s]:cu_np[s + 1]])
            lens.append(int(cu_np[s + 1] - cu_np[s]))
        k, v = torch.cat(ks), torch.cat(vs)
        cu = synth.cu_from_lens(lens)
        q = q[list(seqs)]
    return synth.bits(q), synth.bits(k), synth.bits(v), cu.numpy()


def oracle_step(c: DecodeCase, step: int = 0, seqs=None):
    """Reference results for the live lengths at `step` (optionally for a
    subset of the sequences)."""
    q, k, v, cu = oracle_inputs(c, step, seqs)
    return ora.forward(c.op, q, None, k, v, cu)


def oracle_attend_on(c: DecodeCase, step: int, sel: np.ndarray, cnt: np.ndarray, seqs=None):
    """The reference's attention over a given selection (rows of `sel` /
    `cnt` in the order of `seqs`): how a step's output is checked when its
    selection is a correct one other than the reference's (a near-tie)."""
    q, k, v, cu = oracle_inputs(c, step, seqs)
    max_sel = c.w.topk + c.w.window // c.w.block_size
    sel = np.ascontiguousarray(sel[..., :max_sel], dtype=np.int32)
    return ora.sparse_attend(c.op, q, None, k, v, cu, sel, np.ascontiguousarray(cnt, np.int32))


def check_decode(c: DecodeCase, step: int, g: dict, seqs=None, tag: str = ""):
    """Every check of a fused decode step `g` (gpu_decode_step's results) at
    `step` against the reference, on the listed sequences (all by default):
      * block importance within 1e-4 relative of the reference's;
      * the selection is the rule applied to the step's own fp32 scores,
        bit for bit (every sequence, not only the listed ones);
      * the selection equals the reference's outside the near-tie band;
      * the fused output against the reference's attention on the step's
        own exported selection (always valid: a near-tie makes either set
        correct, and the output is then the attention on the set taken);
      * the fused output against the reference's output directly when the
        selections agree;
      * the stand-alone attention (nosa_sparse_attend) on the reference's
        own selection against the reference's output, for the listed rows
        (the other rows keep the step's own selection).
    Returns the number of near-tie exemptions.  Nothing is skipped."""
    lens = live_lens(c, step)
    rows = list(range(c.B)) if seqs is None else list(seqs)
    o = oracle_step(c, step, seqs=seqs)
    sub = {k: g[k][rows] for k in ("sel", "cnt", "scores", "out", "lse")}
    lens_s = [lens[s] for s in rows]
    compare_scores(sub["scores"], o["scores"], lens_s, c.w)
    check_selection_rule(g["sel"], g["cnt"], g["scores"], lens, c.w)
    ex = compare_selection(sub["sel"], sub["cnt"], o["sel"], o["cnt"], o["scores"], lens_s, c.w)
    oo, ol = oracle_attend_on(c, step, sub["sel"], sub["cnt"], seqs)
    compare_outputs(sub["out"], sub["lse"], oo, ol, tag + " fused (own set)")
    if ex == 0:
        compare_outputs(sub["out"], sub["lse"], o["out"], o["lse"], tag + " fused")
    sel_all = g["sel"].copy()
    cnt_all = g["cnt"].copy()
    n = min(sel_all.shape[-1], o["sel"].shape[-1])
    for i, s in enumerate(rows):
        sel_all[s] = -1
        sel_all[s, ..., :n] = o["sel"][i, ..., :n]
        cnt_all[s] = o["cnt"][i]
    out, lse = gpu_attend(c, step, sel_all, cnt_all)
    compare_outputs(out[rows], lse[rows], o["out"], o["lse"], tag + " attend(oracle set)")
    log(f"{tag}: step {step} ok on sequences {rows if seqs is not None else 'all'} "
        f"(tie exemptions {ex})")
    return o, ex


def local_blocks(w: synth.Workload) -> int:
    """Blocks of the top-k budget forced before the window (locality share)."""
    return math.floor(w.locality * w.topk + 0.5)


def compare_selection(gsel, gcnt, osel, ocnt, oscores, lens, w: synth.Workload):
    """Returns the number of rows where the near-tie exemption was used; raises
    AssertionError on any other disagreement."""
    # the locality share is forced like the window: tie analysis over the
    # earlier candidates and the query-aware part of the budget
    k_loc = local_blocks(w)
    wb = w.window // w.block_size + k_loc
    exempt = 0
    B, _, Hkv, _ = osel.shape
    for s in range(B):
        nb = (lens[s] + w.block_size - 1) // w.block_size
        ncand = max(nb - wb, 0)
        for g in range(Hkv):
            n = int(ocnt[s, 0, g])
            assert int(gcnt[s, 0, g]) == n, (s, g, int(gcnt[s, 0, g]), n)
            a = gsel[s, 0, g, :n].tolist()
            b = osel[s, 0, g, :n].tolist()
            assert np.all(gsel[s, 0, g, n:] == -1), (s, g)
            assert a == sorted(a) and len(set(a)) == n, (s, g, a)
            if a == b:
                continue
            k = min(w.topk - k_loc, ncand)
            sc = oscores[s, 0, g, :ncand]
            order = sorted(range(ncand), key=lambda x: (-sc[x], x))
            kth = sc[order[k - 1]]
            nxt = sc[order[k]] if k < ncand else -np.inf
            gap = abs(kth - nxt) / max(abs(kth), abs(nxt))
            assert gap < TIE_BAND, (s, g, "selection differs outside the tie band", gap)
            diff = set(a) ^ set(b)
            for x in diff:
                assert x < ncand, (s, g, "window differs", x)
                assert abs(sc[x] - kth) <= TIE_BAND * abs(kth), (s, g, x, sc[x], kth)
            exempt += 1
    return exempt


def check_selection_rule(gsel, gcnt, gscores, lens, w: synth.Workload):
    """The fused step's selection is exactly the selection rule applied to its
    own reported block scores (fp32, as the kernel compared them): the
    top-k of the blocks before the forced ones by (score descending, block
    ascending), then the forced blocks, ascending.  Bit-exact, ties included,
    at any size: the selector is checked apart from the rounding of the
    scores, which compare_scores bounds against the reference."""
    k_loc = local_blocks(w)
    wb = w.window // w.block_size + k_loc
    B, _, Hkv, max_sel = gsel.shape
    for s in range(B):
        nb = (lens[s] + w.block_size - 1) // w.block_size
        ncand = max(nb - wb, 0)
        k = min(w.topk - k_loc, ncand)
        for g in range(Hkv):
            sc = gscores[s, 0, g, :ncand].astype(np.float32)
            order = np.lexsort((np.arange(ncand), -sc.astype(np.float64)))[:k]
            want = sorted(order.tolist()) + list(range(ncand, nb))
            n = int(gcnt[s, 0, g])
            assert n == len(want), (s, g, n, len(want))
            got = gsel[s, 0, g, :n].tolist()
            assert got == want, (s, g, "selection is not the rule on the step's own scores")
            assert np.all(gsel[s, 0, g, n:] == -1), (s, g)


def compare_outputs(gout, glse, oout, olse, what=""):
    err = np.abs(gout.astype(np.float64) - oout)
    assert np.isfinite(gout).all(), what
    mx, mean = float(err.max()), float(err.mean())
    assert mx <= OUT_MAX_ABS and mean <= OUT_MEAN_ABS, (what, mx, mean)
    lerr = np.abs(glse.astype(np.float64) - olse)
    assert float(lerr.max()) <= 1e-3 * max(1.0, float(np.abs(olse).max())), (what, lerr.max())
    return mx, mean


def compare_scores(gscores, oscores, lens, w: synth.Workload):
    B, _, Hkv, _ = oscores.shape
    worst = 0.0
    for s in range(B):
        nb = (lens[s] + w.block_size - 1) // w.block_size
        g = gscores[s, 0, :, :nb].astype(np.float64)
        o = oscores[s, 0, :, :nb]
        fin = np.isfinite(o)
        assert np.array_equal(fin, np.isfinite(g)), s
        if fin.any():
            floor = 1e-6 * float(np.abs(o[fin]).max())
            rel = np.abs(g[fin] - o[fin]) / (np.abs(o[fin]) + floor)
            worst = max(worst, float(rel.max()))
        assert np.all(np.isneginf(gscores[s, 0, :, nb:])), s
    assert worst <= TIE_BAND, worst
    return worst
