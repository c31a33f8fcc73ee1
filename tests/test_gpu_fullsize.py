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

from helpers import (TIE_BAND, build_kc, check_decode, oracle_attend_on, check_selection_rule, compare_outputs,
                     compare_selection, gpu_decode_step, gpu_kc_logical, live_lens, log, make_case,
                     oracle_step)

pytestmark = pytest.mark.gpu


def _check_step(c, step, seqs=None, tag=""):
    g = gpu_decode_step(c, step)
    o, _ = check_decode(c, step, g, seqs=seqs, tag=tag)
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
    """The 64K batch-16 workload (32/8 heads, top-k 96) at two consecutive
    steps (the first appends a pooled key): sequences 0, 5, 10 and 15 against
    the reference at each step; every sequence's selection against the rule
    on its own scores, its sizes, window and planted blocks."""
    log("case: decode-b16-64k, sequences 0, 5, 10, 15 at steps 0 and 1")
    w = synth.config(4)
    w.extra_tokens = 1
    c = make_case(w, gen_device="cuda")
    build_kc(c, [L - 1 for L in w.lens])
    for step in (0, 1):
        g, _ = _check_step(c, step, seqs=[0, 5, 10, 15], tag="c4")
        lens = live_lens(c, step)
        for s in range(w.batch):
            nb = (lens[s] + 63) // 64
            for gi in range(w.num_kv_heads):
                n = g["cnt"][s, 0, gi]
                sel = g["sel"][s, 0, gi, :n]
                assert n == min(nb, w.topk + 16)
                assert np.all(np.diff(sel) > 0) and sel[-1] == nb - 1
                assert set(range(nb - 16, nb)) <= set(sel.tolist())
                assert set(c.inp["planted"][s * w.num_kv_heads + gi]) <= set(sel.tolist())
        assert np.isfinite(g["out"]).all() and np.isfinite(g["lse"]).all()
    torch.cuda.empty_cache()


def test_decode_window_beside_long_scoring_varlen():
    """32/8 heads, batch 16, long and short sequences mixed: the attention
    launch is full, so the window pages ride in the scoring launch, a page
    per wave of four-page workgroups (long contexts use the 8-tile scoring
    kernel); the short sequences leave window waves and whole window
    workgroups empty.  Sequences 0 and 12..15 against the reference, every
    sequence's selection against the rule on its own scores."""
    lens = [40000] * 12 + [100, 700, 1000, 2100]
    log(f"case: window beside the scoring, lengths {lens}")
    w = synth.Workload(lens=lens, num_q_heads=32, num_kv_heads=8, topk=96, planted=2, seed=21,
                       window=1024, name="t")
    c = make_case(w, gen_device="cuda")
    build_kc(c, [L - 1 for L in w.lens])
    g, _ = _check_step(c, 0, seqs=[0, 12, 13, 14, 15], tag="window-beside-scoring")
    check_selection_rule(g["sel"], g["cnt"], g["scores"], live_lens(c, 0), w)
    assert np.isfinite(g["out"]).all() and np.isfinite(g["lse"]).all()
    torch.cuda.empty_cache()


def test_offload_b8_16k_steps():
    """The 16K batch-8 workload over an offloaded KV cache, as the bench runs
    it: four steps with correlated queries, each bit-identical to the step
    over device pools, the cache holding every pick; sequences 0 and 7 of the
    first step against the reference."""
    import math
    from helpers import cu_dev
    from test_gpu_offload import Offloaded
    from block_sparse_attention_nosa_amd import nosa
    log("case: decode-b8-16k offloaded, 4 steps")
    w = synth.config(2)
    c = make_case(w, gen_device="cuda")
    build_kc(c, [L - 1 for L in w.lens])
    off = Offloaded(c, recent=20, cap=128)
    off.kc.copy_(c.pg["kc_pool"])
    gen = torch.Generator(device="cuda").manual_seed(5)
    qf = c.inp["q"].float()
    B, maxL = c.B, max(w.lens) + 3
    for t in range(4):
        if t:
            qf = 0.9 * qf + math.sqrt(0.19) * torch.randn(qf.shape, generator=gen, device="cuda")
        q = qf.to(torch.bfloat16)
        lens = [L + t for L in w.lens]
        cu = cu_dev(lens)
        off.fill_ring(lens)
        res = []
        for fn in ("dev", "off"):
            out = torch.empty(B, 16, 128, device="cuda")
            lse = torch.empty(B, 16, device="cuda")
            sel = torch.empty(B, 1, 2, 80, dtype=torch.int32, device="cuda")
            cnt = torch.empty(B, 1, 2, dtype=torch.int32, device="cuda")
            if fn == "dev":
                ws = torch.zeros(nosa.nosa_workspace_size(c.p, B, 1, maxL), dtype=torch.uint8,
                                 device="cuda")
                nosa.nosa_decode_step(c.p, c.kv, q, cu, B, maxL, out, lse, ws, sel_idx=sel,
                                      sel_count=cnt)
            else:
                ws = torch.zeros(nosa.nosa_offload_workspace_size(c.p, B, maxL, 128),
                                 dtype=torch.uint8, device="cuda")
                nosa.nosa_offload_decode_step(c.p, off.okv, q, cu, B, maxL, out, lse, ws,
                                              sel_idx=sel, sel_count=cnt)
            torch.cuda.synchronize()
            res.append((out, lse, sel, cnt))
        for a, b in zip(res[0], res[1]):
            assert torch.equal(a, b), t
        sel, cnt = res[1][2].cpu().numpy(), res[1][3].cpu().numpy()
        cmap = off.map.cpu().numpy()
        for s in range(B):
            nb = (lens[s] + 63) // 64
            for g in range(2):
                picks = {int(x) for x in sel[s, 0, g, :cnt[s, 0, g]] if x < nb - 16}
                assert picks <= set(cmap[s, g].tolist()), (t, s, g)
        if t == 0:
            rows = [0, 7]
            o = oracle_step(c, 0, seqs=rows)
            ex = compare_selection(sel[rows], cnt[rows], o["sel"], o["cnt"], o["scores"],
                                   [lens[s] for s in rows], w)
            gout, glse = res[1][0].cpu().numpy()[rows], res[1][1].cpu().numpy()[rows]
            # on the step's own set always; on the reference's when they agree
            oo, ol = oracle_attend_on(c, 0, sel[rows], cnt[rows], seqs=rows)
            compare_outputs(gout, glse, oo, ol, "offloaded c2 (own set)")
            if ex == 0:
                compare_outputs(gout, glse, o["out"], o["lse"], "offloaded c2")
        log(f"offloaded c2: step {t} ok")


def test_layer_step_b8_16k_from_hidden():
    """The 16K batch-8 workload from hidden states of width 2048 (the bench's
    --front 2048): q, k, v within one bf16 ulp of the reference, the step on
    them bit-identical to the decode step on the same queries, sequences 0 and
    3 against the reference forward on the reference's q, k, v."""
    from helpers import cu_dev
    from test_gpu_front import _close_bf16, _slot_values
    from block_sparse_attention_nosa_amd import nosa
    log("case: decode-b8-16k from hidden states")
    w = synth.config(2)
    c = make_case(w, gen_device="cuda")
    lens = list(w.lens)
    build_kc(c, [L - 1 for L in lens])
    hidden, B, maxL = 2048, c.B, max(lens)
    gen = torch.Generator().manual_seed(11)
    wt = (torch.randn(20 * 128, hidden, generator=gen) / hidden ** 0.5).to(torch.bfloat16)
    x = torch.randn(B, hidden, generator=gen).to(torch.bfloat16)
    packed = torch.empty_like(wt.cuda())
    nosa.nosa_pack_qkv_weights(c.p, hidden, wt.cuda(), packed)
    q_out = torch.empty(B, 16, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.empty(B, 16, 128, device="cuda")
    lse = torch.empty(B, 16, device="cuda")
    sel = torch.empty(B, 1, 2, 80, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, 1, 2, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nosa.nosa_workspace_size(c.p, B, 1, maxL), dtype=torch.uint8, device="cuda")
    cu = cu_dev(lens)
    nosa.nosa_layer_decode_step(c.p, nosa.front_params(hidden), c.kv, x.cuda(), packed, cu, B,
                                maxL, q_out, out, lse, ws, sel_idx=sel, sel_count=cnt)
    torch.cuda.synchronize()
    pos = np.array([L - 1 for L in lens], np.int32)
    oq, ok, ov = ora.qkv_rope(c.op, synth.bits(x), synth.bits(wt), pos)
    _close_bf16(synth.bits(q_out.cpu()), oq, "q")
    gk, gv = _slot_values(c, lens)
    _close_bf16(gk, ok, "k")
    _close_bf16(gv, ov, "v")
    # the same step on the front end's queries
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    build_kc(c, [L - 1 for L in lens])
    nosa.nosa_decode_step(c.p, c.kv, q_out, cu, B, maxL, out2, lse2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    # the reference on its own q, k, v for sequences 0 and 3
    rows = [0, 3]
    k, v, cu_l = synth.packed_live(c.inp, w, 0)
    kb, vb = synth.bits(k.cpu()).copy(), synth.bits(v.cpu()).copy()
    cu_np = cu_l.numpy()
    ks, vs, ls = [], [], []
    for s in rows:
        kk, vv = kb[cu_np[s]:cu_np[s + 1]].copy(), vb[cu_np[s]:cu_np[s + 1]].copy()
        kk[-1], vv[-1] = ok[s], ov[s]
        ks.append(kk)
        vs.append(vv)
        ls.append(lens[s])
    o = ora.forward(c.op, oq[rows], None, np.concatenate(ks), np.concatenate(vs),
                    synth.cu_from_lens(ls).numpy())
    g_sel, g_cnt = sel.cpu().numpy()[rows], cnt.cpu().numpy()[rows]
    ex = compare_selection(g_sel, g_cnt, o["sel"], o["cnt"], o["scores"], ls, w)
    g_out, g_lse = out.cpu().numpy()[rows], lse.cpu().numpy()[rows]
    # the step's output against the reference's attention on the step's own
    # set (always), and on the reference's set when the two agree
    oo, ol = ora.sparse_attend(c.op, oq[rows], None, np.concatenate(ks), np.concatenate(vs),
                               synth.cu_from_lens(ls).numpy(), g_sel, g_cnt)
    compare_outputs(g_out, g_lse, oo, ol, "layer step c2 (own set)")
    if ex == 0:
        compare_outputs(g_out, g_lse, o["out"], o["lse"], "layer step c2")
    log(f"layer step c2: ok (tie exemptions {ex})")


def test_prompt_32k_sampled_query_blocks():
    """The bench's whole-prompt workload (32768 tokens, chunks of 4096): query
    blocks 0, 100, 300 and 511 against the reference, each solved as its own
    problem cut after the block's last query (nothing later is visible).  The
    stand-alone chain over the same prompt supplies the selection the prompt
    prefill shares: its importance and selection against the reference (near-
    tie band), and the prompt's output against the reference's attention on
    that selection for every sampled block, and against the reference's
    output where the selections agree.  Every sampled block is compared."""
    from helpers import cu_dev
    from test_gpu_prefill import check_rows, compare_out, gpu_prefill
    from block_sparse_attention_nosa_amd import nosa
    log("case: whole-prompt prefill, 32768 tokens, sampled query blocks")
    L = 32768
    w = synth.Workload(lens=[L], q_lens=[L], topk=64, planted=0, seed=1000 + L, name="prompt")
    c = make_case(w, gen_device="cuda")
    q = c.inp["q"]
    out = torch.empty(L, 16, 128, device="cuda")
    lse = torch.empty(L, 16, device="cuda")
    ws = torch.zeros(nosa.nosa_prefill_sparse_workspace_size(c.p, 1, L, 4096), dtype=torch.uint8,
                     device="cuda")
    nosa.nosa_prefill_sparse(c.p, c.kv, q, cu_dev([L]), 1, L, 4096, out, lse, ws)
    torch.cuda.synchronize()
    go, gl = out.cpu().numpy(), lse.cpu().numpy()
    assert np.isfinite(go).all()
    del ws
    g, _ = gpu_prefill(c)  # the pooled keys are the prompt prefill's own
    compared = 0
    for r in (0, 100, 300, 511):
        p_last = 64 * r + 63
        kk = synth.bits(c.inp["k"][:p_last + 1])
        vv = synth.bits(c.inp["v"][:p_last + 1])
        qq = synth.bits(q[64 * r:64 * r + 64])
        cu_q, cu_k = np.array([0, 64], np.int32), np.array([0, p_last + 1], np.int32)
        o = ora.forward(c.op, qq, cu_q, kk, vv, cu_k)
        e = check_rows(g, o, [(0, r, 0, 0)], w, f"prompt r{r}")
        rows = slice(64 * r, 64 * r + 64)
        oo, ol = ora.sparse_attend(c.op, qq, cu_q, kk, vv, cu_k, g["sel"][:, r:r + 1],
                                   g["cnt"][:, r:r + 1])
        compare_out(go[rows], gl[rows], oo, ol, f"prompt r{r} (own set)")
        if e == 0:
            compare_out(go[rows], gl[rows], o["out"], o["lse"], f"prompt r{r}")
        compared += 1
        log(f"prompt 32K q-block {r}: ok (tie exemptions {e})")
    assert compared == 4
