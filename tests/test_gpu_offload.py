"""GPU parity of the decode step over an offloaded KV cache
(nosa_offload_decode_step): K/V pages in pinned host memory, the recent pages
in a device ring, the top-k picks in a per-(sequence, KV head) block cache.
Each step must equal the ordinary decode step over device pools holding the
same pages bit for bit (same selection, same outputs), the cache must hold
every pick afterwards with contents equal to the host pages, and exactly the
picks missing from the cache before the step must have been read from host
memory.  The last step of each case is also checked against the oracle."""
import numpy as np
import pytest
import torch

from block_sparse_attention_nosa_amd import nosa, synth
from oracle import oracle as ora

from helpers import (build_kc, compare_outputs, compare_selection, cu_dev, local_blocks, log,
                     make_case)

pytestmark = pytest.mark.gpu


def _wl(lens, hq=16, hkv=2, topk=8, planted=2, seed=11, locality=0.0, extra=24):
    w = synth.Workload(lens=list(lens), num_q_heads=hq, num_kv_heads=hkv, topk=topk,
                       planted=planted, seed=seed, name="offload", locality=locality)
    w.extra_tokens = extra
    return w


class Offloaded:
    """Host pools, recent ring, block cache and pooled keys of an offloaded
    copy of a case's paged cache."""

    def __init__(self, c, recent, cap):
        pg = c.pg
        self.c, self.recent, self.cap = c, recent, cap
        B, Hkv = c.B, c.w.num_kv_heads
        page = pg["k_pool"].shape[-1]
        self.k_host = torch.empty(pg["k_pool"].shape, dtype=torch.bfloat16, pin_memory=True)
        self.v_host = torch.empty(pg["v_pool"].shape, dtype=torch.bfloat16, pin_memory=True)
        self.k_host.copy_(pg["k_pool"].cpu())
        self.v_host.copy_(pg["v_pool"].cpu())
        self.kc = pg["kc_pool"].clone()  # pooled keys: device, its own copy
        self.k_ring = torch.zeros(B, recent, Hkv, page, dtype=torch.bfloat16, device="cuda")
        self.v_ring = torch.zeros_like(self.k_ring)
        self.cache_k = torch.zeros(B, Hkv, cap, page, dtype=torch.bfloat16, device="cuda")
        self.cache_v = torch.zeros_like(self.cache_k)
        self.map = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device="cuda")
        # no initial contents needed: poison them
        self.used = torch.full((B, Hkv, cap), 12345, dtype=torch.int32, device="cuda")
        self.okv = nosa.offload_kv(self.k_host, self.v_host, self.kc, pg["block_table"],
                                   self.k_ring, self.v_ring, self.cache_k, self.cache_v, self.map,
                                   self.used)

    def fill_ring(self, lens):
        """The last `recent` blocks of each sequence into their ring slots."""
        pg, R = self.c.pg, self.recent
        for s, L in enumerate(lens):
            nb = (L + 63) // 64
            for b in range(max(0, nb - R), nb):
                page = int(pg["block_table"][s, b])
                self.k_ring[s, b % R] = pg["k_pool"][page]
                self.v_ring[s, b % R] = pg["v_pool"][page]


def _outputs(c, lens):
    W = c.w
    max_sel = W.topk + W.window // 64
    return dict(out=torch.full((c.B, W.num_q_heads, 128), float("nan"), device="cuda"),
                lse=torch.full((c.B, W.num_q_heads), float("nan"), device="cuda"),
                sel=torch.full((c.B, 1, W.num_kv_heads, max_sel), -7, dtype=torch.int32,
                               device="cuda"),
                cnt=torch.full((c.B, 1, W.num_kv_heads), -7, dtype=torch.int32, device="cuda"))


def _run(c, off, steps, queries, tag):
    w = c.w
    k_loc = local_blocks(w)
    wb = w.window // 64 + k_loc
    build_kc(c, [L - 1 for L in w.lens])
    off.kc.copy_(c.pg["kc_pool"])
    total_fetch = 0
    for t in range(steps):
        lens = [L + t for L in w.lens]
        maxL = max(lens)
        q = queries[t % len(queries)]
        a, b = _outputs(c, lens), _outputs(c, lens)
        ws = torch.zeros(nosa.nosa_workspace_size(c.p, c.B, 1, maxL), dtype=torch.uint8,
                         device="cuda")
        nosa.nosa_decode_step(c.p, c.kv, q, cu_dev(lens), c.B, maxL, a["out"], a["lse"], ws,
                              sel_idx=a["sel"], sel_count=a["cnt"])
        off.fill_ring(lens)
        old_map = off.map.cpu().numpy().copy()
        old_used = off.used.cpu().numpy().copy()
        fetch = torch.full((c.B, w.num_kv_heads), -7, dtype=torch.int32, device="cuda")
        wso = torch.zeros(nosa.nosa_offload_workspace_size(c.p, c.B, maxL, off.cap),
                          dtype=torch.uint8, device="cuda")
        nosa.nosa_offload_decode_step(c.p, off.okv, q, cu_dev(lens), c.B, maxL, b["out"], b["lse"],
                                      wso, sel_idx=b["sel"], sel_count=b["cnt"], fetch_count=fetch)
        torch.cuda.synchronize()
        ga = {k: v.cpu().numpy() for k, v in a.items()}
        gb = {k: v.cpu().numpy() for k, v in b.items()}
        for k in ("sel", "cnt", "out", "lse"):
            assert np.array_equal(ga[k], gb[k]), (tag, t, k)
        new_map = off.map.cpu().numpy()
        new_used = off.used.cpu().numpy()
        fetch = fetch.cpu().numpy()
        for s, L in enumerate(lens):
            nb = (L + 63) // 64
            ncand = max(nb - wb, 0)
            for g in range(w.num_kv_heads):
                n = int(gb["cnt"][s, 0, g])
                picks = {int(x) for x in gb["sel"][s, 0, g, :n] if x < ncand}
                held = {int(x) for x in new_map[s, g] if x >= 0}
                assert picks <= held, (tag, t, s, g, sorted(picks - held))
                before = {int(x) for x in old_map[s, g] if x >= 0}
                assert int(fetch[s, g]) == len(picks - before), (tag, t, s, g)
                # blocks that stay cached keep their slot
                for slot, blk in enumerate(old_map[s, g]):
                    if blk in picks:
                        assert new_map[s, g, slot] == blk, (tag, t, s, g, slot)
                # the misses went to the free slots picked least recently
                # (empty slots first, then by length at the last pick, then by slot)
                free = [x for x in range(off.cap) if old_map[s, g, x] not in picks]
                order = sorted(free, key=lambda x: (-1 if old_map[s, g, x] < 0
                                                    else int(old_used[s, g, x]), x))
                nmiss = len(picks - before)
                filled = {x for x in free if new_map[s, g, x] != old_map[s, g, x]
                          or (old_map[s, g, x] < 0 and new_map[s, g, x] >= 0)}
                assert filled == set(order[:nmiss]), (tag, t, s, g)
                for x in range(off.cap):  # lengths at the last pick
                    if new_map[s, g, x] in picks:
                        assert new_used[s, g, x] == L, (tag, t, s, g, x)
                    elif new_map[s, g, x] >= 0:
                        assert new_used[s, g, x] == old_used[s, g, x], (tag, t, s, g, x)
                total_fetch += int(fetch[s, g])
        # cache contents equal the host pages
        table = c.pg["block_table"].cpu().numpy()
        for s in range(c.B):
            for g in range(w.num_kv_heads):
                for slot, blk in enumerate(new_map[s, g]):
                    if blk < 0:
                        continue
                    page = int(table[s, blk])
                    assert torch.equal(off.cache_k[s, g, slot].cpu(), off.k_host[page, g]), \
                        (tag, t, s, g, slot)
                    assert torch.equal(off.cache_v[s, g, slot].cpu(), off.v_host[page, g]), \
                        (tag, t, s, g, slot)
    # pooled keys appended through the ring equal those of the ordinary steps
    assert torch.equal(off.kc, c.pg["kc_pool"]), tag
    # the last step against the oracle
    lens = [L + steps - 1 for L in w.lens]
    k, v, cu = synth.packed_live(c.inp, w, steps - 1)
    q = queries[(steps - 1) % len(queries)].cpu()
    o = ora.forward(c.op, synth.bits(q), None, synth.bits(k), synth.bits(v), cu.numpy())
    ex = compare_selection(gb["sel"], gb["cnt"], o["sel"], o["cnt"], o["scores"], lens, w)
    # on the step's own set always; on the reference's when they agree
    oo, ol = ora.sparse_attend(c.op, synth.bits(q), None, synth.bits(k), synth.bits(v), cu.numpy(),
                               gb["sel"][..., :w.topk + w.window // 64], gb["cnt"])
    compare_outputs(gb["out"], gb["lse"], oo, ol, tag + " (own set)")
    if ex == 0:
        compare_outputs(gb["out"], gb["lse"], o["out"], o["lse"], tag)
    log(f"{tag}: ok, {steps} steps, {total_fetch} blocks read from host, tie exemptions {ex}")
    return total_fetch


def _queries(c, n, seed):
    gen = torch.Generator().manual_seed(seed)
    qs = [c.inp["q"].cuda()]
    for _ in range(n - 1):
        qs.append(torch.randn(c.inp["q"].shape, generator=gen).to(torch.bfloat16).cuda())
    return qs


@pytest.mark.parametrize("lens,cap_extra", [([3000, 4100, 2200], 0), ([3000, 4100, 2200], 40),
                                            ([1100, 5000], 5)])
def test_offload_matches_device_pools(lens, cap_extra):
    log(f"case: offload lens {lens} cache topk+{cap_extra}")
    c = make_case(_wl(lens, seed=len(lens) + cap_extra))
    off = Offloaded(c, recent=17, cap=c.w.topk + cap_extra)
    # three queries in turn: the cache sees repeats as well as changes
    _run(c, off, 12, _queries(c, 3, 5), f"offload {lens} +{cap_extra}")


def test_offload_repeated_query_fetches_nothing_new():
    log("case: offload, same query every step")
    c = make_case(_wl([6000, 3500], topk=12, seed=3, extra=8))
    off = Offloaded(c, recent=16, cap=12)
    q = c.inp["q"].cuda()
    first = _run(c, off, 1, [q], "offload first step")
    assert first == sum(min(12, (L + 63) // 64 - 16) for L in c.w.lens) * c.w.num_kv_heads
    # the same query again: picks can shift only where the sequence grew
    off.map.fill_(-1)
    total = _run(c, off, 6, [q], "offload same query")
    assert total <= first + 6 * c.B * c.w.num_kv_heads


@pytest.mark.parametrize("hq,hkv,topk,locality", [(32, 8, 10, 0.0), (12, 3, 16, 0.5),
                                                   (16, 2, 64, 0.25)])
def test_offload_heads_and_locality(hq, hkv, topk, locality):
    log(f"case: offload heads {hq}/{hkv} topk {topk} locality {locality}")
    c = make_case(_wl([5200, 2600], hq=hq, hkv=hkv, topk=topk, seed=hq + topk,
                      locality=locality))
    k_loc = local_blocks(c.w)
    recent = max(2, 1024 // 64 + k_loc)
    off = Offloaded(c, recent=recent, cap=topk - k_loc)
    _run(c, off, 6, _queries(c, 2, 9), f"offload {hq}/{hkv} k{topk} loc{locality}")


def test_offload_no_window_locality_only():
    """Window 0 with a locality share: the forced set is the 8 local blocks
    (the current token's block among them), served from the ring; the other
    8 picks go through the cache."""
    log("case: offload, no window, locality 0.5")
    w = synth.Workload(lens=[3000, 4500], topk=16, window=0, planted=2, seed=17, name="offload",
                       locality=0.5)
    w.extra_tokens = 24
    c = make_case(w)
    off = Offloaded(c, recent=8, cap=8)
    _run(c, off, 6, _queries(c, 2, 21), "offload window 0")


def test_offload_short_sequences():
    log("case: offload short sequences (no candidates)")
    c = make_case(_wl([40, 700, 1030], seed=2, planted=0))
    off = Offloaded(c, recent=16, cap=8)
    _run(c, off, 5, _queries(c, 2, 4), "offload short")


def test_offload_errors():
    c = make_case(_wl([3000]))
    off = Offloaded(c, recent=16, cap=8)
    ws = torch.zeros(nosa.nosa_offload_workspace_size(c.p, 1, 3000, 8), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(1, 16, 128, device="cuda")
    q = c.inp["q"].cuda()
    call = lambda okv: nosa.nosa_offload_decode_step(c.p, okv, q, cu_dev([3000]), 1, 3000, out,
                                                     None, ws)
    # pageable host memory cannot be read by the device
    pageable = torch.zeros(off.k_host.shape, dtype=torch.bfloat16)
    bad = nosa.offload_kv(pageable, off.v_host, off.kc, c.pg["block_table"], off.k_ring,
                          off.v_ring, off.cache_k, off.cache_v, off.map, off.used)
    with pytest.raises(nosa.NosaError) as e:
        call(bad)
    assert e.value.status == 2
    # a device tensor is not host memory either
    bad = nosa.offload_kv(c.pg["k_pool"], off.v_host, off.kc, c.pg["block_table"], off.k_ring,
                          off.v_ring, off.cache_k, off.cache_v, off.map, off.used)
    with pytest.raises(nosa.NosaError) as e:
        call(bad)
    assert e.value.status == 2
    call(off.okv)  # and the good one works
    torch.cuda.synchronize()
