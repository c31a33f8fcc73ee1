"""HIP-graph capture of the entry points (the bench times graph replays): each
call is captured once, then replayed several times with other eager GPU work
in between; every replay must reproduce the eager result bit for bit.  The
library records no memset and no host synchronisation, so a captured call is
the same sequence of kernels as an eager one."""
import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth

from helpers import build_kc, cu_dev, log, make_case

pytestmark = pytest.mark.gpu


def _replays(fn, outs, n=4):
    """fn(): enqueue the call; outs: tensors it writes.  Eager result, then n
    replays of a captured call with unrelated eager work between them."""
    fn()
    torch.cuda.synchronize()
    ref = [o.clone() for o in outs]
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    junk = torch.randn(1 << 20, device="cuda")
    for i in range(n):
        for o in outs:
            o.fill_(float("nan") if o.is_floating_point() else -7)
        junk.mul_(1.0001).add_(i)  # eager work between replays
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        for o, r in zip(outs, ref):
            assert torch.equal(o, r), i
    return ref


def _wl(lens, **kw):
    return synth.Workload(lens=list(lens), topk=kw.pop("topk", 8), planted=2, seed=13,
                          name="graph", **kw)


def test_decode_step_graph():
    log("case: decode step in a graph")
    c = make_case(_wl([3000, 4100, 2047]))
    lens = c.w.lens
    build_kc(c, [L - 1 for L in lens])
    B, maxL = c.B, max(lens)
    out = torch.empty(B, 16, 128, device="cuda")
    lse = torch.empty(B, 16, device="cuda")
    sel = torch.empty(B, 1, 2, 8 + 16, dtype=torch.int32, device="cuda")
    cnt = torch.empty(B, 1, 2, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nosa.nosa_workspace_size(c.p, B, 1, maxL), dtype=torch.uint8, device="cuda")
    q, cu = c.inp["q"].cuda(), cu_dev(lens)
    _replays(lambda: nosa.nosa_decode_step(c.p, c.kv, q, cu, B, maxL, out, lse, ws, sel_idx=sel,
                                           sel_count=cnt), [out, lse, sel, cnt])


def test_prompt_prefill_graph():
    log("case: whole-prompt prefill in a graph")
    w = synth.Workload(lens=[2600, 700], q_lens=[2600, 700], topk=8, seed=3, name="graph")
    c = make_case(w)
    B, maxL = c.B, max(w.lens)
    q, cu = c.inp["q"].cuda(), cu_dev(w.lens)
    out = torch.empty(q.shape[0], 16, 128, device="cuda")
    lse = torch.empty(q.shape[0], 16, device="cuda")
    ws = torch.zeros(nosa.nosa_prefill_sparse_workspace_size(c.p, B, maxL, 512),
                     dtype=torch.uint8, device="cuda")
    _replays(lambda: nosa.nosa_prefill_sparse(c.p, c.kv, q, cu, B, maxL, 512, out, lse, ws),
             [out, lse])


def test_offload_and_layer_step_graph():
    log("case: offloaded step and layer step in graphs")
    from test_gpu_offload import Offloaded
    c = make_case(_wl([3000, 2000]))
    lens = c.w.lens
    B, maxL = c.B, max(lens)
    build_kc(c, [L - 1 for L in lens])
    off = Offloaded(c, recent=16, cap=12)
    off.fill_ring(lens)
    off.kc.copy_(c.pg["kc_pool"])
    q, cu = c.inp["q"].cuda(), cu_dev(lens)
    out = torch.empty(B, 16, 128, device="cuda")
    lse = torch.empty(B, 16, device="cuda")
    ws = torch.zeros(nosa.nosa_offload_workspace_size(c.p, B, maxL, 12), dtype=torch.uint8,
                     device="cuda")
    # the first call fills the cache; the replays hit it and must give the same result
    _replays(lambda: nosa.nosa_offload_decode_step(c.p, off.okv, q, cu, B, maxL, out, lse, ws),
             [out, lse])
    # front end + decode step from hidden states
    hidden = 512
    gen = torch.Generator().manual_seed(2)
    wt = (torch.randn(20 * 128, hidden, generator=gen) / hidden ** 0.5).to(torch.bfloat16).cuda()
    packed = torch.empty_like(wt)
    nosa.nosa_pack_qkv_weights(c.p, hidden, wt, packed)
    x = torch.randn(B, hidden, generator=gen).to(torch.bfloat16).cuda()
    front = nosa.front_params(hidden)
    q_out = torch.empty(B, 16, 128, dtype=torch.bfloat16, device="cuda")
    ws2 = torch.zeros(nosa.nosa_workspace_size(c.p, B, 1, maxL), dtype=torch.uint8, device="cuda")
    _replays(lambda: nosa.nosa_layer_decode_step(c.p, front, c.kv, x, packed, cu, B, maxL, q_out,
                                                 out, lse, ws2), [q_out, out, lse])
