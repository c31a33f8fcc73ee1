"""Seeded synthetic inputs for the NOSA decode / chunked-prefill step.

This module only *builds inputs*: random bf16 queries and keys/values, planted
high-scoring blocks, varlen lengths and the paged KV layout.  It holds none of
the method's arithmetic, so the CPU reference and the HIP library can both be
fed from it without sharing any computation.

Recipe (the same for every workload):
  * values are float32 draws from N(0, 1) on a seeded torch generator, rounded
    to bf16 (round-to-nearest-even); draw order: K, V, q, planted positions,
    page permutation;
  * a planted block of KV head g has all of its keys shifted by 0.5 * qhat_g
    before rounding, where qhat_g = sqrt(d) * unit(sum of the group's query
    heads) of the first query of the sequence: a logit margin of about 2 after
    the 1/sqrt(d) scale; planted blocks are drawn uniformly, without
    replacement, among blocks that stay outside the local window;
  * pages hold block_size tokens; each sequence's blocks are laid out in page
    order and then the whole pool is put through a seeded random permutation.

Packed layouts (what the CPU reference reads):
  q [total_q][Hq][d], k / v [total_k][Hkv][d]  (bf16), cu_seqlens int32.
Paged layouts (what the library reads): one page holds block_size tokens of
one KV head; pages are [num_pages][Hkv][page elements] and the elements of a
page are in the library's operand order (see page_index below):
  k_pool  [num_pages][Hkv][block_size * d]
  v_pool  [num_pages][Hkv][block_size * d]
  kc_pool [num_pages][Hkv][block_size / stride * d]
  block_table [B][max_blocks] int32 (unused entries 0).
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import List, Optional

import torch


@dataclass
class Workload:
    """A batch of sequences sharing one attention shape."""
    lens: List[int]                  # KV length per sequence (incl. the current token)
    num_q_heads: int = 16
    num_kv_heads: int = 2
    head_dim: int = 128
    block_size: int = 64
    kernel: int = 32
    stride: int = 16
    topk: int = 64
    window: int = 1024
    locality: float = 0.0            # share of topk given to the blocks nearest the window
    planted: int = 0                 # planted blocks per (sequence, KV head)
    q_lens: Optional[List[int]] = None  # queries per sequence (None: one, decode)
    seed: int = 0
    extra_tokens: int = 0            # tokens pre-written beyond lens (multi-step decode)
    name: str = ""
    meta: dict = field(default_factory=dict)

    @property
    def batch(self) -> int:
        return len(self.lens)

    @property
    def group(self) -> int:
        return self.num_q_heads // self.num_kv_heads


def _bf16(x: torch.Tensor) -> torch.Tensor:
    return x.to(torch.bfloat16)


def cu_from_lens(lens, device="cpu") -> torch.Tensor:
    cu = [0]
    for n in lens:
        cu.append(cu[-1] + int(n))
    return torch.tensor(cu, dtype=torch.int32, device=device)


def make_inputs(w: Workload, device="cpu") -> dict:
    """Packed bf16 tensors for workload w (deterministic in w.seed)."""
    gen = torch.Generator(device=device)
    gen.manual_seed(int(w.seed))
    Hq, Hkv, d, G = w.num_q_heads, w.num_kv_heads, w.head_dim, w.group
    stored = [L + w.extra_tokens for L in w.lens]
    total_k = sum(stored)
    q_lens = w.q_lens if w.q_lens is not None else [1] * w.batch
    total_q = sum(q_lens)
    k = torch.randn(total_k, Hkv, d, generator=gen, device=device, dtype=torch.float32)
    v = torch.randn(total_k, Hkv, d, generator=gen, device=device, dtype=torch.float32)
    q = _bf16(torch.randn(total_q, Hq, d, generator=gen, device=device, dtype=torch.float32))
    cu_k_store = cu_from_lens(stored, device)
    cu_q = cu_from_lens(q_lens, device)
    planted = []
    if w.planted > 0:
        qf = q.float()
        for s, L in enumerate(w.lens):
            Lq = q_lens[s]
            first_q_pos = L - Lq
            # blocks wholly before the window of the first query stay candidates
            nb_first = first_q_pos // w.block_size + 1
            ncand = nb_first - w.window // w.block_size
            row = int(cu_q[s])
            for g in range(Hkv):
                if ncand <= 0:
                    planted.append([])
                    continue
                n = min(w.planted, ncand)
                blocks = torch.randperm(ncand, generator=gen, device=device)[:n]
                blocks = sorted(int(b) for b in blocks)
                planted.append(blocks)
                qsum = qf[row, g * G:(g + 1) * G].sum(0)
                qhat = math.sqrt(d) * qsum / qsum.norm()
                base = int(cu_k_store[s])
                for b in blocks:
                    t0 = base + b * w.block_size
                    k[t0:t0 + w.block_size, g] += 0.5 * qhat
    k = _bf16(k)
    v = _bf16(v)
    return dict(q=q, k=k, v=v, cu_k_store=cu_k_store, cu_q=cu_q, q_lens=q_lens,
                stored_lens=stored, planted=planted, gen=gen)


def cu_k_at(w: Workload, step: int, device="cpu") -> torch.Tensor:
    """cu_seqlens over the *stored* layout is fixed; the live lengths at a decode
    step are lens + step.  Returns the live lengths as cu_seqlens of the live
    tokens (a length descriptor only: the paged kernels never use the offsets
    to address K/V)."""
    return cu_from_lens([L + step for L in w.lens], device)


def packed_live(inp: dict, w: Workload, step: int = 0):
    """Packed K/V/cu of the first lens+step tokens of each sequence (for the CPU
    reference at a given decode step)."""
    ks, vs = [], []
    for s, L in enumerate(w.lens):
        base = int(inp["cu_k_store"][s])
        ks.append(inp["k"][base:base + L + step])
        vs.append(inp["v"][base:base + L + step])
    return torch.cat(ks), torch.cat(vs), cu_from_lens([L + step for L in w.lens])


def page_index(kind: str, block_size: int = 64, d: int = 128, stride: int = 16) -> torch.Tensor:
    """For each stored element of a page, the index of the element it holds
    in the logical page ([token][channel] for "k" and "v", [slot][channel]
    for "kc"), so that stored = logical.flatten()[page_index(kind)].

    Stored offsets, element e of 8 (all pages of 64 tokens x 128 channels):
      k : (((4t + st) * 4 + kq) * 16 + m) * 8 + e holds channel 32st + 8kq + e
          of token 32(t // 2) + 8(m // 4) + 4(t % 2) + m % 4;
      v : (((8u + nt) * 4 + kq) * 16 + r) * 8 + e holds token 32u + 8kq + e of
          channel 16nt + r;
      kc: (c8 * 4 + j) * 8 + e holds channel 8c8 + e of slot j.
    """
    assert block_size == 64 and d == 128 and stride == 16
    o = torch.arange(block_size * d if kind != "kc" else block_size // stride * d)
    e = o & 7
    if kind == "k":
        m, kq, st, t = (o >> 3) & 15, (o >> 7) & 3, (o >> 9) & 3, o >> 11
        tok = 32 * (t >> 1) + 8 * (m >> 2) + 4 * (t & 1) + (m & 3)
        return tok * d + 32 * st + 8 * kq + e
    if kind == "v":
        r, kq, nt, u = (o >> 3) & 15, (o >> 7) & 3, (o >> 9) & 7, o >> 12
        return (32 * u + 8 * kq + e) * d + 16 * nt + r
    if kind == "kc":
        j, c8 = (o >> 3) & 3, o >> 5
        return j * d + 8 * c8 + e
    raise ValueError(kind)


def to_paged(inp: dict, w: Workload, permute: bool = True, device=None) -> dict:
    """Scatter the packed K/V into the paged pools (see the module docstring)."""
    k, v = inp["k"], inp["v"]
    device = device or k.device
    bs, Hkv, d = w.block_size, w.num_kv_heads, w.head_dim
    nbs = [(n + bs - 1) // bs for n in inp["stored_lens"]]
    num_pages = max(1, sum(nbs))
    max_blocks = max(1, max(nbs))
    if permute:
        gen = inp["gen"]
        perm = torch.randperm(num_pages, generator=gen, device=gen.device).to(device)
    else:
        perm = torch.arange(num_pages, device=device)
    table = torch.zeros(w.batch, max_blocks, dtype=torch.int32, device=device)
    k_pool = torch.zeros(num_pages, Hkv, bs * d, dtype=torch.bfloat16, device=device)
    v_pool = torch.zeros(num_pages, Hkv, bs * d, dtype=torch.bfloat16, device=device)
    kidx = page_index("k", bs, d, w.stride).to(device)
    vidx = page_index("v", bs, d, w.stride).to(device)
    logical = 0
    for s, n in enumerate(inp["stored_lens"]):
        base = int(inp["cu_k_store"][s])
        pad = nbs[s] * bs - n
        ks = k[base:base + n].to(device)
        vs = v[base:base + n].to(device)
        if pad:
            ks = torch.cat([ks, torch.zeros(pad, Hkv, d, dtype=ks.dtype, device=device)])
            vs = torch.cat([vs, torch.zeros(pad, Hkv, d, dtype=vs.dtype, device=device)])
        pages = perm[logical:logical + nbs[s]]
        table[s, :nbs[s]] = pages.to(torch.int32)
        # [nb, bs, Hkv, d] -> logical pages [nb, Hkv, bs * d] -> stored order
        kb = ks.view(nbs[s], bs, Hkv, d).permute(0, 2, 1, 3).reshape(nbs[s], Hkv, bs * d)
        vb = vs.view(nbs[s], bs, Hkv, d).permute(0, 2, 1, 3).reshape(nbs[s], Hkv, bs * d)
        k_pool[pages.long()] = kb[:, :, kidx]
        v_pool[pages.long()] = vb[:, :, vidx]
        logical += nbs[s]
    kc_pool = torch.zeros(num_pages, Hkv, bs // w.stride * d, dtype=torch.bfloat16,
                          device=device)
    return dict(k_pool=k_pool, v_pool=v_pool, kc_pool=kc_pool, block_table=table,
                max_blocks=max_blocks, num_pages=num_pages)


def bits(t: torch.Tensor):
    """bf16 tensor -> numpy uint16 bit patterns (host)."""
    return t.detach().contiguous().cpu().view(torch.int16).numpy().view("uint16")


# --------------------------------------------------------------- workloads ---

def config(n: int, seed: Optional[int] = None) -> Workload:
    """The five workloads of the NOSA decode/prefill measurements (sizes as
    named; seed 1000 + n unless given)."""
    sd = 1000 + n if seed is None else seed
    if n == 1:   # batch 1, 4K context, top-k 16, 4 planted blocks per KV head
        return Workload(lens=[4096], topk=16, planted=4, seed=sd, name="decode-b1-4k")
    if n == 2:   # NOSA-1B shape, batch 8, 16K context, top-k 64, 256 decode steps
        return Workload(lens=[16384 + 1] * 8, topk=64, planted=8, seed=sd, extra_tokens=255,
                        name="decode-b8-16k")
    if n == 3:   # varlen batch 32, lengths uniform in [4096, 32768], permuted pages
        g = torch.Generator().manual_seed(sd)
        lens = torch.randint(4096, 32768 + 1, (32,), generator=g).tolist()
        return Workload(lens=lens, topk=64, planted=0, seed=sd, name="decode-varlen-b32")
    if n == 4:   # 8B-scale GQA, batch 16, 64K context, top-k 96
        return Workload(lens=[65536] * 16, num_q_heads=32, num_kv_heads=8, topk=96, planted=8,
                        seed=sd, name="decode-b16-64k-gqa4")
    if n == 5:   # chunked sparse prefill: 2048 queries at the end of 131072 tokens
        return Workload(lens=[131072], q_lens=[2048], topk=64, planted=0, seed=sd,
                        name="prefill-2048-of-131072")
    raise ValueError(f"no workload {n}")
