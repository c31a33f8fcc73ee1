"""GPU parity beyond 2048 blocks per sequence, up to the library's limit of
8192 blocks (524288 tokens): contexts of hundreds of thousands of tokens, the
range the NOSA pages give for the method.  Past 2048 blocks the selector keeps
the candidates beyond its register rounds in LDS, the attention launch reads
the block-table row and the importance of those blocks through LDS, and at
8192 blocks a selection workgroup holds 64 KB of dynamic LDS.  Checked: the
decode step (pooled keys bit-exact, importance, the selection rule on the
step's own scores, the reference's selection outside the near-tie band,
outputs on both selections), nosa_block_scores in decode mode, the stand-alone
selection on shared scores with heavy exact ties, and the chunked prefill's
importance, selection and attention."""
import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth
from oracle import oracle as ora

from helpers import (build_kc, check_decode, compare_scores, cu_dev, gpu_decode_step,
                     gpu_kc_logical, live_lens, log, make_case, workspace)

pytestmark = pytest.mark.gpu


def _wl(lens, hq=16, hkv=2, topk=64, planted=4, seed=1, window=1024, q_lens=None):
    return synth.Workload(lens=list(lens), num_q_heads=hq, num_kv_heads=hkv, topk=topk,
                          planted=planted, seed=seed, window=window, q_lens=q_lens, name="long")


def _scores_only(c, lens):
    """nosa_block_scores in decode mode (cu_seqlens_q NULL): the importance of
    the query at position L-1 over the pooled keys of all L tokens."""
    B, maxL = c.B, max(lens)
    max_nb = (maxL + 63) // 64
    scores = torch.full((B, 1, c.w.num_kv_heads, max_nb), float("nan"), device="cuda")
    nosa.nosa_block_scores(c.p, c.kv, c.inp["q"].cuda(), None, cu_dev(lens), B, 1, maxL, scores,
                           workspace(c, maxL))
    torch.cuda.synchronize()
    return scores.cpu().numpy()


@pytest.mark.parametrize("hq,hkv,L,topk", [(16, 2, 200_000, 64), (8, 1, 300_000, 96),
                                           (16, 2, 524_288, 64), (8, 1, 524_288, 1000)])
def test_decode_step_long_context(hq, hkv, L, topk):
    log(f"case: long decode heads {hq}/{hkv} L={L} topk={topk}")
    c = make_case(_wl([L], hq=hq, hkv=hkv, topk=topk, seed=L % 1000 + hq), gen_device="cuda")
    lens = live_lens(c, 0)
    build_kc(c, [x - 1 for x in lens])
    g = gpu_decode_step(c, 0)
    o, _ = check_decode(c, 0, g, tag=f"long {hq}/{hkv} L={L}")
    nc = ora.num_keys(L, c.op)
    assert np.array_equal(gpu_kc_logical(c, 0, nc), o["kc"][0, :, :nc])
    for gi in range(hkv):
        chosen = set(g["sel"][0, 0, gi, :g["cnt"][0, 0, gi]].tolist())
        assert set(c.inp["planted"][gi]) <= chosen, gi
    # the stand-alone importance in decode mode: the fused step's own scores
    # (same kernels), bit for bit, after the step appended the last key
    sc = _scores_only(c, lens)
    assert np.array_equal(sc, g["scores"])
    torch.cuda.empty_cache()


def test_block_scores_decode_mode_varlen():
    """nosa_block_scores with cu_seqlens_q NULL on a varlen batch from one
    block to beyond 2048 blocks: against the reference's importance (1e-4
    relative), -inf past each sequence's blocks."""
    lens = [1, 40, 1000, 5000, 140_000]
    log(f"case: block scores, decode mode, lengths {lens}")
    c = make_case(_wl(lens, hq=12, hkv=3, planted=1, seed=77), gen_device="cuda")
    build_kc(c, lens)
    sc = _scores_only(c, lens)
    q, k, v = synth.bits(c.inp["q"]), synth.bits(c.inp["k"]), synth.bits(c.inp["v"])
    cu = synth.cu_from_lens(lens).numpy()
    kc = ora.compress_keys(c.op, k, cu)
    os_ = ora.block_scores(c.op, q, None, kc, cu)
    worst = compare_scores(sc, os_, lens, c.w)
    log(f"block scores decode mode: worst relative error {worst:.2e}")
    torch.cuda.empty_cache()


@pytest.mark.parametrize("lens,topk", [([524_288, 300_000], 64), ([524_288, 131_000], 3000)])
def test_select_long_shared_scores(lens, topk):
    """The stand-alone selection on fp32 scores shared with the reference,
    values in a handful of levels (heavy exact ties: lower block index wins),
    up to 8192 blocks (16 candidate rounds of the eight-wave selector, 8 of
    them read from LDS): identical sets and counts."""
    log(f"case: select on shared scores, lengths {lens}, topk {topk}")
    rng = np.random.default_rng(topk)
    max_nb = (max(lens) + 63) // 64
    B = len(lens)
    sc = rng.integers(0, 7, (B, 1, 2, max_nb)).astype(np.float32) * np.float32(0.125)
    sc[1, 0, 1, :] = 0.5  # all tied
    for s, L in enumerate(lens):
        sc[s, 0, :, (L + 63) // 64:] = -np.inf
    p = nosa.params(topk=topk)
    op = ora.Params(topk=topk)
    cu = synth.cu_from_lens(lens)
    osel, ocnt = ora.select_blocks(op, sc.astype(np.float64), None, cu.numpy())
    sel = torch.empty(B, 1, 2, topk + 16, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, 1, 2, dtype=torch.int32, device="cuda")
    nosa.nosa_select_blocks(p, torch.as_tensor(sc).cuda(), None, cu.cuda(), B, 1, max(lens), sel,
                            cnt)
    torch.cuda.synchronize()
    assert np.array_equal(cnt.cpu().numpy(), ocnt)
    assert np.array_equal(sel.cpu().numpy(), osel)


def test_prefill_long_context():
    """A 130-query chunk (three query blocks, the last ragged) at the end of
    a 200000-token context (3125 blocks): importance, selection and
    attention of every query block against the reference."""
    from test_gpu_prefill import _full
    log("case: prefill, 130 queries over 200000 tokens")
    c = make_case(_wl([200_000], topk=64, planted=0, seed=9, q_lens=[130]), gen_device="cuda")
    _full(c, "pf long 200000")
    torch.cuda.empty_cache()
