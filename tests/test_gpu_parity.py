"""GPU (gfx950) parity of every entry point of the C ABI against the CPU
reference, on seeded synthetic inputs, small enough for the reference to finish
in seconds but spanning several tiles, ragged tails and the degenerate cases."""
import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth
from oracle import oracle as ora

from helpers import (DecodeCase, build_kc, check_decode, compare_outputs, compare_selection,
                     cu_dev, gpu_decode_step, gpu_kc_logical, live_lens, log, make_case,
                     oracle_attend_on, oracle_step, workspace)

pytestmark = pytest.mark.gpu


def _wl(lens, hq=16, hkv=2, topk=16, planted=2, seed=7, window=1024, locality=0.0):
    return synth.Workload(lens=list(lens), num_q_heads=hq, num_kv_heads=hkv, topk=topk,
                          planted=planted, seed=seed, window=window, name="t",
                          locality=locality)


def _full_check(c: DecodeCase, step=0, tag=""):
    lens = live_lens(c, step)
    build_kc(c, [L - 1 for L in lens])
    g = gpu_decode_step(c, step)
    # pooled keys: bit-exact (the step appended the last one); then every
    # check of the step (scores, selection rule, selection, outputs on both
    # selections)
    o, ex = check_decode(c, step, g, tag=tag)
    for s, L in enumerate(lens):
        nc = ora.num_keys(L, c.op)
        assert np.array_equal(gpu_kc_logical(c, s, nc), o["kc"][s, :, :nc]), (tag, s)
    return g, o, ex


def test_mfma_lane_layout_through_dense_attention():
    """top-k covering every block: the fused step is dense attention; any
    mistake in the MFMA operand layouts shows up here first."""
    log("case: dense G=8 L=700")
    c = make_case(_wl([700], topk=100, planted=0))
    _full_check(c, tag="dense")


@pytest.mark.parametrize("hq,hkv", [(16, 2), (32, 8), (8, 8), (16, 1), (12, 3)])
def test_decode_step_head_groups(hq, hkv):
    log(f"case: heads {hq}/{hkv}")
    c = make_case(_wl([3000, 1500, 4100], hq=hq, hkv=hkv, topk=8, seed=hq * 100 + hkv))
    _full_check(c, tag=f"{hq}/{hkv}")


@pytest.mark.parametrize("hq,hkv,L", [(16, 1, 40000), (8, 1, 70000)])
def test_decode_step_logits_beyond_lds(hq, hkv, L):
    """A group of 16 heads over 40K tokens (8 over 70K) has more logits than
    one workgroup's LDS holds next to its other arrays: the step keeps them in
    the workspace instead of in LDS."""
    log(f"case: logits beyond LDS, heads {hq}/{hkv}, L={L}")
    c = make_case(_wl([L, 1000], hq=hq, hkv=hkv, topk=32, planted=3, seed=L + hq))
    _full_check(c, tag=f"zglobal {hq}/{hkv}")


def test_empty_budget_no_topk_no_window():
    """top-k 0 and no window: nothing is selected; the fused step and the
    stand-alone attention (whose block lists then have no entries; a
    one-entry buffer is passed, and must not be read) give out = 0 and
    lse = -inf, as the reference does."""
    log("case: top-k 0, window 0")
    lens = [300, 2000, 64 * 9 + 5]
    c = make_case(_wl(lens, topk=0, window=0, planted=0, seed=3))
    build_kc(c, [L - 1 for L in lens])
    g = gpu_decode_step(c, 0)
    o = oracle_step(c, 0)
    assert np.all(g["cnt"] == 0) and np.all(o["cnt"] == 0)
    assert np.all(o["out"] == 0) and np.all(np.isneginf(o["lse"]))
    assert np.all(g["out"] == 0) and np.all(np.isneginf(g["lse"]))
    W = c.w
    out = torch.full((c.B, W.num_q_heads, W.head_dim), float("nan"), device="cuda")
    lse = torch.full((c.B, W.num_q_heads), float("nan"), device="cuda")
    sel_d = torch.full((1,), 7, dtype=torch.int32, device="cuda")  # would be a block id if read
    cnt_d = torch.zeros((c.B, 1, W.num_kv_heads), dtype=torch.int32, device="cuda")
    nosa.nosa_sparse_attend(c.p, c.kv, c.inp["q"].to("cuda"), None, cu_dev(lens), c.B, 1, max(lens),
                            sel_d, cnt_d, out, lse, workspace(c, max(lens)))
    torch.cuda.synchronize()
    assert torch.all(out == 0).item() and torch.all(torch.isneginf(lse)).item()


@pytest.mark.parametrize("hq,hkv,lens", [(16, 2, [3000, 20000]), (8, 1, [70000])])
def test_decode_step_tied_scores(hq, hkv, lens):
    """A zero query: every logit is 0, so the block importances tie (up to
    the rounding of their sums) and the pick between tied blocks falls to
    the lower index; from tens to over a thousand candidate blocks (one and
    several candidate rounds per selector thread)."""
    log(f"case: tied scores, heads {hq}/{hkv}, lengths {lens}")
    c = make_case(_wl(lens, hq=hq, hkv=hkv, topk=24, planted=0, seed=5))
    c.inp["q"] = torch.zeros_like(c.inp["q"])
    _full_check(c, tag="tied")


@pytest.mark.parametrize("lens", [
    [1], [17], [31], [32], [33], [63, 64, 65], [1023, 1024, 1025],
    [1088, 1089, 1090, 1151], [2047, 2048, 2049], [5000, 40, 3333, 64 * 17 + 5]])
def test_decode_step_lengths(lens):
    log(f"case: lengths {lens}")
    c = make_case(_wl(lens, topk=4, planted=0, seed=sum(lens)))
    _full_check(c, tag=str(lens))


@pytest.mark.parametrize("batch,hq,hkv", [(96, 16, 2), (40, 32, 8)])
def test_decode_step_large_batch(batch, hq, hkv):
    """Many (sequence, KV head) pairs: 192 and 320 of them, more attention
    workgroups than the chip holds at once, so the window pages go to the
    scoring launch or share the attention launch with longer top-k
    workgroups."""
    log(f"case: batch {batch}, heads {hq}/{hkv}")
    g = torch.Generator().manual_seed(batch)
    lens = torch.randint(900, 3200, (batch,), generator=g).tolist()
    c = make_case(_wl(lens, hq=hq, hkv=hkv, topk=6, planted=1, seed=batch + hq))
    _full_check(c, tag=f"batch {batch}")


@pytest.mark.parametrize("topk", [0, 1, 3, 64, 500])
def test_decode_step_topk(topk):
    log(f"case: topk {topk}")
    c = make_case(_wl([4096, 2500], topk=topk, planted=3, seed=topk + 1))
    _full_check(c, tag=f"topk{topk}")


@pytest.mark.parametrize("window", [0, 64, 512, 4096])
def test_decode_step_window(window):
    log(f"case: window {window}")
    c = make_case(_wl([3000, 700], topk=5, planted=0, seed=window + 3, window=window))
    _full_check(c, tag=f"win{window}")


@pytest.mark.parametrize("locality,topk", [(0.75, 64), (0.5, 5), (1.0, 16), (0.25, 96)])
def test_decode_step_locality(locality, topk):
    """Locality constraint: round(locality * topk) forced blocks before the
    window, the rest by importance (varlen batch, both window placements)."""
    log(f"case: locality {locality} topk {topk}")
    c = make_case(_wl([9000, 2500, 700], topk=topk, planted=2, seed=int(locality * 40) + topk,
                      locality=locality))
    _full_check(c, tag=f"loc{locality}/{topk}")


def test_planted_blocks_found_on_gpu():
    log("case: 4K planted")
    w = synth.config(1)
    c = make_case(w)
    g, o, _ = _full_check(c, tag="c1")
    for gi in range(2):
        chosen = set(g["sel"][0, 0, gi, :g["cnt"][0, 0, gi]].tolist())
        assert set(c.inp["planted"][gi]) <= chosen


def test_compress_keys_full_incremental_and_append():
    log("case: compress keys")
    lens = [5000, 31, 32, 1000, 64 * 7 + 17]
    c = make_case(_wl(lens, topk=4, planted=0, seed=11))
    o = ora.compress_keys(c.op, synth.bits(c.inp["k"]), synth.cu_from_lens(lens).numpy())
    build_kc(c, lens)                              # full build
    torch.cuda.synchronize()
    full = [gpu_kc_logical(c, s, ora.num_keys(L, c.op)) for s, L in enumerate(lens)]
    for s, L in enumerate(lens):
        assert np.array_equal(full[s], o[s, :, :ora.num_keys(L, c.op)]), s
    # wipe and rebuild in two increments: first 60% of each sequence, then the rest
    c.pg["kc_pool"].zero_()
    first = [int(L * 0.6) for L in lens]
    build_kc(c, first)
    build_kc(c, lens, valid=first)
    torch.cuda.synchronize()
    for s, L in enumerate(lens):
        assert np.array_equal(gpu_kc_logical(c, s, ora.num_keys(L, c.op)), full[s]), s


def test_multi_step_decode_appends_keys():
    """32 consecutive steps with appends: the pooled keys equal a full rebuild
    and every step matches the reference."""
    log("case: multi-step")
    w = _wl([1500, 2001], topk=6, planted=2, seed=5)
    w.extra_tokens = 40
    c = make_case(w)
    build_kc(c, [L - 1 for L in w.lens])
    for step in range(33):
        g = gpu_decode_step(c, step)
        if step % 8 == 0 or step == 32:
            check_decode(c, step, g, tag=f"step{step}")
    lens = live_lens(c, 32)
    kcs = [gpu_kc_logical(c, s, ora.num_keys(L, c.op)) for s, L in enumerate(lens)]
    build_kc(c, lens)
    torch.cuda.synchronize()
    for s, L in enumerate(lens):
        assert np.array_equal(kcs[s], gpu_kc_logical(c, s, ora.num_keys(L, c.op))), s


def test_select_bit_exact_on_shared_scores():
    """Both sides take the decision on the same fp32 values: identical sets,
    including exact ties (which must go to the lower block index)."""
    log("case: select on shared scores")
    rng = np.random.default_rng(3)
    lens = [5000, 1100, 64 * 40, 3]
    w = _wl(lens, topk=9)
    p = nosa.params(topk=9)
    op = ora.Params(topk=9)
    max_nb = (max(lens) + 63) // 64
    sc = rng.integers(0, 6, (len(lens), 1, 2, max_nb)).astype(np.float32)  # heavy ties
    sc[1, 0, 1, :] = 0.25                                                 # all tied
    for s, L in enumerate(lens):
        sc[s, 0, :, (L + 63) // 64:] = -np.inf
    cu = synth.cu_from_lens(lens)
    osel, ocnt = ora.select_blocks(op, sc.astype(np.float64), None, cu.numpy())
    sel = torch.empty(len(lens), 1, 2, 9 + 16, dtype=torch.int32, device="cuda")
    cnt = torch.empty(len(lens), 1, 2, dtype=torch.int32, device="cuda")
    nosa.nosa_select_blocks(p, torch.as_tensor(sc).cuda(), None, cu.cuda(), len(lens), 1,
                            max(lens), sel, cnt)
    torch.cuda.synchronize()
    assert np.array_equal(cnt.cpu().numpy(), ocnt)
    assert np.array_equal(sel.cpu().numpy(), osel)
    del w


def test_page_permutation_and_determinism():
    """Results are bitwise independent of where the pages sit in the pool, and
    bitwise repeatable."""
    log("case: permutation")
    w = _wl([4000, 2222], topk=7, planted=2, seed=9)
    c1 = make_case(w, permute=True)
    c2 = make_case(w, permute=False)
    outs = []
    for c in (c1, c2, c1):
        build_kc(c, [L - 1 for L in w.lens])
        outs.append(gpu_decode_step(c, 0))
    for key in ("out", "lse", "sel", "cnt", "scores"):
        assert np.array_equal(outs[0][key], outs[1][key], equal_nan=True), key
        assert np.array_equal(outs[0][key], outs[2][key], equal_nan=True), key


def test_varlen_batch_equals_single_sequences():
    log("case: batch vs single")
    lens = [3000, 1200, 4500]
    w = _wl(lens, topk=5, planted=2, seed=19)
    c = make_case(w)
    build_kc(c, [L - 1 for L in lens])
    full = gpu_decode_step(c, 0)
    for s, L in enumerate(lens):
        ws = _wl([L], topk=5, planted=0, seed=1)
        cs = make_case(ws)
        # same tensors for sequence s
        base = int(c.inp["cu_k_store"][s])
        cs.inp["k"][:] = c.inp["k"][base:base + L]
        cs.inp["v"][:] = c.inp["v"][base:base + L]
        cs.inp["q"][:] = c.inp["q"][s:s + 1]
        cs.pg.update(synth.to_paged(cs.inp, ws, device="cuda"))
        cs.kv = nosa.paged_kv(cs.pg["k_pool"], cs.pg["v_pool"], cs.pg["kc_pool"],
                              cs.pg["block_table"])
        build_kc(cs, [L - 1])
        one = gpu_decode_step(cs, 0)
        n = full["cnt"][s, 0]
        assert np.array_equal(n, one["cnt"][0, 0])
        for g in range(2):
            assert np.array_equal(full["sel"][s, 0, g, :n[g]], one["sel"][0, 0, g, :n[g]])
        # Same selection; the output may differ by the bf16 rounding of P: the
        # pages a wave accumulates follow the plan (workgroups per pair),
        # which depends on the batch, and P is rounded relative to the wave's
        # running maximum.  2^-9 relative on weights summing to 1, times |v|
        # <= ~4, bounds it well below 1e-3.
        np.testing.assert_allclose(full["out"][s], one["out"][0], rtol=0, atol=1e-3)


def test_stream_argument_is_honoured():
    log("case: side stream")
    c = make_case(_wl([2000], topk=4, planted=1, seed=23))
    build_kc(c, [1999])
    ref = gpu_decode_step(c, 0)
    st = torch.cuda.Stream()
    out = torch.empty(1, 16, 128, device="cuda")
    lse = torch.empty(1, 16, device="cuda")
    ws = workspace(c, 2000)
    torch.cuda.synchronize()
    with torch.cuda.stream(st):
        nosa.nosa_decode_step(c.p, c.kv, c.inp["q"].cuda(), cu_dev([2000]), 1, 2000, out, lse, ws,
                              stream=st)
    st.synchronize()
    assert np.array_equal(out.cpu().numpy(), ref["out"])


def test_workspace_reuse_across_sizes():
    """One workspace (sized for the largest call) serves consecutive calls of
    different sizes: nothing a call leaves behind changes the next one.
    Every call is checked against the reference (on its own exported
    selection, and on the reference's when they agree), and the two calls on
    the large batch are bitwise identical."""
    log("case: workspace reuse")
    big = make_case(_wl([5000, 3000, 4000], topk=6, planted=2, seed=31))
    small = make_case(_wl([1500], topk=6, planted=1, seed=32))
    ws = workspace(big, 5000)
    results = []
    for c in (big, small, big):
        lens = live_lens(c, 0)
        build_kc(c, [L - 1 for L in lens])
        out = torch.full((c.B, 16, 128), float("nan"), device="cuda")
        lse = torch.full((c.B, 16), float("nan"), device="cuda")
        sel = torch.full((c.B, 1, 2, 6 + 16), -7, dtype=torch.int32, device="cuda")
        cnt = torch.full((c.B, 1, 2), -7, dtype=torch.int32, device="cuda")
        nosa.nosa_decode_step(c.p, c.kv, c.inp["q"].cuda(), cu_dev(lens), c.B, max(lens), out,
                              lse, ws, sel_idx=sel, sel_count=cnt)
        torch.cuda.synchronize()
        g = dict(out=out.cpu().numpy(), lse=lse.cpu().numpy(), sel=sel.cpu().numpy(),
                 cnt=cnt.cpu().numpy())
        o = oracle_step(c, 0)
        ex = compare_selection(g["sel"], g["cnt"], o["sel"], o["cnt"], o["scores"], lens, c.w)
        oo, ol = oracle_attend_on(c, 0, g["sel"], g["cnt"])
        compare_outputs(g["out"], g["lse"], oo, ol, f"reuse B={c.B} (own set)")
        if ex == 0:
            compare_outputs(g["out"], g["lse"], o["out"], o["lse"], f"reuse B={c.B}")
        results.append(g)
    for key in ("out", "lse", "sel", "cnt"):
        assert np.array_equal(results[0][key], results[2][key]), key
