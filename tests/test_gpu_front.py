"""GPU parity of the attention front end (nosa_pack_qkv_weights,
nosa_qkv_rope_append, nosa_layer_decode_step): QKV projection of each
sequence's current token, rotary encoding of q and k, k and v written into the
token's page slot, then the decode step on those queries.  q, k and v are
compared with the reference's bf16 values (GPU: fp32 accumulation, so at most
one bf16 unit in the last place apart, nearly all identical); the layer step's
selection and outputs with the reference forward run on the reference's own
q, k and v."""
import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth
from oracle import oracle as ora

from helpers import (build_kc, compare_outputs, compare_selection, cu_dev, log, make_case)

pytestmark = pytest.mark.gpu


def _wl(lens, hq=16, hkv=2, topk=8, seed=21, planted=0):
    w = synth.Workload(lens=list(lens), num_q_heads=hq, num_kv_heads=hkv, topk=topk,
                       planted=planted, seed=seed, name="front")
    return w


def _weights(c, hidden, seed):
    gen = torch.Generator().manual_seed(seed)
    rows = (c.w.num_q_heads + 2 * c.w.num_kv_heads) * 128
    w = (torch.randn(rows, hidden, generator=gen) / hidden ** 0.5).to(torch.bfloat16)
    x = torch.randn(c.B, hidden, generator=gen).to(torch.bfloat16)
    return w, x


def _packed(c, w, hidden):
    wd = w.cuda()
    packed = torch.empty_like(wd)
    nosa.nosa_pack_qkv_weights(c.p, hidden, wd, packed)
    torch.cuda.synchronize()
    return packed


def _close_bf16(g, o, what):
    """g, o: bf16 bit arrays.  At most one bf16 ulp apart, mostly identical."""
    gv = (g.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    ov = (o.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.isfinite(gv).all(), what
    tol = 2.0 ** -7 * np.maximum(np.abs(gv), np.abs(ov)) + 1e-6
    bad = np.abs(gv - ov) > tol
    assert not bad.any(), (what, int(bad.sum()), float(np.abs(gv - ov).max()))
    same = float((gv == ov).mean())
    assert same > 0.97, (what, same)
    return same


def _slot_values(c, lens):
    """K and V stored in each sequence's slot of position L-1: [B][Hkv][128] bits."""
    kidx = synth.page_index("k").numpy()
    vidx = synth.page_index("v").numpy()
    table = c.pg["block_table"].cpu().numpy()
    kpool = c.pg["k_pool"].cpu().view(torch.int16).numpy().view(np.uint16)
    vpool = c.pg["v_pool"].cpu().view(torch.int16).numpy().view(np.uint16)
    Hkv = c.w.num_kv_heads
    k = np.zeros((c.B, Hkv, 128), np.uint16)
    v = np.zeros((c.B, Hkv, 128), np.uint16)
    for s, L in enumerate(lens):
        page, x = table[s, (L - 1) // 64], (L - 1) % 64
        for g in range(Hkv):
            # stored[o] holds logical element idx[o] = token * 128 + channel
            lk = np.empty(64 * 128, np.uint16)
            lk[kidx] = kpool[page, g]
            lv = np.empty(64 * 128, np.uint16)
            lv[vidx] = vpool[page, g]
            k[s, g] = lk[x * 128:(x + 1) * 128]
            v[s, g] = lv[x * 128:(x + 1) * 128]
    return k, v


def test_pack_layout():
    log("case: packed weight layout")
    c = make_case(_wl([300]))
    hidden = 512
    w, _ = _weights(c, hidden, 1)
    packed = _packed(c, w, hidden).cpu().view(torch.int16).numpy().view(np.uint16)
    wb = w.view(torch.int16).numpy().view(np.uint16)
    nkb = hidden // 256
    idx = np.arange(packed.size)
    e, lane, t = idx % 8, (idx // 8) % 64, (idx // 512) % 8
    kb, T = (idx // 4096) % nkb, idx // (4096 * nkb)
    m, grp = lane % 16, lane // 16
    head, j = T // 8, T % 8
    row = head * 128 + np.where(m < 8, 8 * j + m, 64 + 8 * j + (m - 8))
    col = 256 * kb + 32 * t + 8 * grp + e
    assert np.array_equal(packed.reshape(-1), wb[row, col])


@pytest.mark.parametrize("hq,hkv,hidden,lens,theta,custom", [
    (16, 2, 2048, [3000, 4100, 70, 1, 1025, 2222, 64, 65], 10000.0, False),
    (32, 8, 4096, [5000, 131000], 500000.0, False),
    (12, 3, 768, [900] * 20, 10000.0, True)])
def test_front_matches_reference(hq, hkv, hidden, lens, theta, custom):
    log(f"case: front end heads {hq}/{hkv} hidden {hidden} batch {len(lens)}")
    c = make_case(_wl(lens, hq=hq, hkv=hkv, seed=hq + hidden))
    w, x = _weights(c, hidden, hq + hkv)
    packed = _packed(c, w, hidden)
    f64 = None
    f_dev = None
    if custom:  # a scaled table of angles per pair (as long-context rescalings give)
        f64 = (theta ** (-np.arange(64) * 2.0 / 128)) / np.linspace(1.0, 8.0, 64)
        f32 = f64.astype(np.float32)
        f64 = f32.astype(np.float64)  # the GPU reads float32 values
        f_dev = torch.tensor(f32, device="cuda")
    front = nosa.front_params(hidden, theta, f_dev)
    k_before = c.pg["k_pool"].clone()
    v_before = c.pg["v_pool"].clone()
    q_out = torch.full((c.B, hq, 128), -1, dtype=torch.int16, device="cuda").view(torch.bfloat16)
    nosa.nosa_qkv_rope_append(c.p, front, c.kv, x.cuda(), packed, cu_dev(lens), c.B, max(lens),
                              q_out)
    torch.cuda.synchronize()
    pos = np.array([L - 1 for L in lens], np.int32)
    oq, ok, ov = ora.qkv_rope(c.op, synth.bits(x), synth.bits(w), pos, theta=theta, inv_freq=f64)
    sq = _close_bf16(synth.bits(q_out.cpu()), oq, "q")
    gk, gv = _slot_values(c, lens)
    sk = _close_bf16(gk, ok, "k")
    sv = _close_bf16(gv, ov, "v")
    # nothing else in the pools changed
    table = c.pg["block_table"].cpu().numpy()
    touched = {int(table[s, (L - 1) // 64]) for s, L in enumerate(lens)}
    keep = torch.ones(c.pg["k_pool"].shape[0], dtype=torch.bool)
    keep[sorted(touched)] = False
    assert torch.equal(c.pg["k_pool"][keep.cuda()], k_before[keep.cuda()])
    assert torch.equal(c.pg["v_pool"][keep.cuda()], v_before[keep.cuda()])
    log(f"front end: identical bf16 values q {sq:.4f}, k {sk:.4f}, v {sv:.4f}")


@pytest.mark.parametrize("hq,hkv,topk,lens", [(16, 2, 8, [3000, 4100, 2500]),
                                               (32, 8, 10, [5200, 2600])])
def test_layer_decode_step_matches_reference(hq, hkv, topk, lens):
    log(f"case: layer decode step heads {hq}/{hkv} lens {lens}")
    hidden = 2048
    c = make_case(_wl(lens, hq=hq, hkv=hkv, topk=topk, seed=len(lens) + hq))
    build_kc(c, [L - 1 for L in lens])
    w, x = _weights(c, hidden, 77)
    packed = _packed(c, w, hidden)
    front = nosa.front_params(hidden, 10000.0)
    B, maxL, W = c.B, max(lens), c.w
    q_out = torch.empty(B, hq, 128, dtype=torch.bfloat16, device="cuda")
    out = torch.full((B, hq, 128), float("nan"), device="cuda")
    lse = torch.full((B, hq), float("nan"), device="cuda")
    max_sel = topk + W.window // 64
    sel = torch.full((B, 1, hkv, max_sel), -7, dtype=torch.int32, device="cuda")
    cnt = torch.full((B, 1, hkv), -7, dtype=torch.int32, device="cuda")
    ws = torch.zeros(nosa.nosa_workspace_size(c.p, B, 1, maxL), dtype=torch.uint8, device="cuda")
    nosa.nosa_layer_decode_step(c.p, front, c.kv, x.cuda(), packed, cu_dev(lens), B, maxL, q_out,
                                out, lse, ws, sel_idx=sel, sel_count=cnt)
    torch.cuda.synchronize()
    # the reference: its own q, k, v for the current token, then the forward
    pos = np.array([L - 1 for L in lens], np.int32)
    oq, ok, ov = ora.qkv_rope(c.op, synth.bits(x), synth.bits(w), pos)
    k, v, cu = synth.packed_live(c.inp, W, 0)
    kb, vb = synth.bits(k).copy(), synth.bits(v).copy()
    cu_np = cu.numpy()
    for s in range(B):
        kb[cu_np[s + 1] - 1] = ok[s]
        vb[cu_np[s + 1] - 1] = ov[s]
    o = ora.forward(c.op, oq, None, kb, vb, cu_np)
    g = dict(sel=sel.cpu().numpy(), cnt=cnt.cpu().numpy(), out=out.cpu().numpy(),
             lse=lse.cpu().numpy())
    ex = compare_selection(g["sel"], g["cnt"], o["sel"], o["cnt"], o["scores"], lens, W)
    # the step's output against the reference's attention on the step's own
    # set (always), and on the reference's set when the two agree
    oo, ol = ora.sparse_attend(c.op, oq, None, kb, vb, cu_np, g["sel"], g["cnt"])
    mx, mean = compare_outputs(g["out"], g["lse"], oo, ol, "layer step (own set)")
    log(f"layer step: max abs {mx:.2e}, mean abs {mean:.2e}")
    if ex == 0:
        compare_outputs(g["out"], g["lse"], o["out"], o["lse"], "layer step")
    # the step used the front end's queries: same result as the decode step on q_out
    out2 = torch.full_like(out, float("nan"))
    lse2 = torch.full_like(lse, float("nan"))
    build_kc(c, [L - 1 for L in lens])
    nosa.nosa_decode_step(c.p, c.kv, q_out, cu_dev(lens), B, maxL, out2, lse2, ws)
    torch.cuda.synchronize()
    assert torch.equal(out, out2) and torch.equal(lse, lse2)
    log(f"layer step: ok (tie exemptions {ex})")


def test_front_errors():
    c = make_case(_wl([300]))
    x = torch.zeros(1, 256, dtype=torch.bfloat16, device="cuda")
    w = torch.zeros(20 * 128, 256, dtype=torch.bfloat16, device="cuda")
    q = torch.empty(1, 16, 128, dtype=torch.bfloat16, device="cuda")
    for hidden, status in ((100, 2), (0, 2)):
        with pytest.raises(nosa.NosaError) as e:
            nosa.nosa_qkv_rope_append(c.p, nosa.front_params(hidden), c.kv, x, w,
                                      cu_dev([300]), 1, 300, q)
        assert e.value.status == status
    with pytest.raises(nosa.NosaError) as e:
        nosa.nosa_pack_qkv_weights(c.p, 100, w, w)
    assert e.value.status == 2
