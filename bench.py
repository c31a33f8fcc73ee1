"""Benchmark of the NOSA sparse decode step on one MI355X.

    python bench.py [--gpus 1] [--steps K] [--warmup W] [--config 2]

Workload (default, config 2): the NOSA-1B attention shape -- 16 query / 2 KV
heads, head_dim 128 -- decode batch 8 at 16K context, top-k 64 blocks + the
1024-token window, 8 planted blocks per KV head, 256 decode steps that append
to K/V and the pooled keys.  Inputs are seeded synthetic bf16 N(0, 1) values
generated on the GPU.  Eight independent layer caches (136 MB each) are used
in rotation so consecutive steps cannot be served from the 256 MB Infinity
Cache; step i runs layer i % 8 at decode position (i // 8) % 256.

A step is the whole hot path for the batch: append the pooled key completed by
the current token, score the pooled keys, pool the scores into block
importance, select top-k + window, attend over the kept blocks, merge.  The
timed region is K such steps back to back on one stream (replays of a HIP
graph of the steps), bracketed by device synchronisations; inputs are
resident in HBM before it starts.

Printed: one JSON line with the throughput (decode tokens/s = batch / step
time), the roofline of the dominant kernel (the sparse attention, timed with
HIP events around its own launches on the launch stream) and the CPU
reference's throughput on a bounded sample of the same workload.

Traffic counters (kept out of the timed run):
    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o run --output-format csv -- python bench.py --pmc-probe
    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o run --output-format csv -- python bench.py --pmc-probe
    python bench.py --pmc-summary DIR_F DIR_W > profiles/attention-decode-b8-16k_traffic.md
The probe runs a plain copy of 256 MiB (calibration: bytes per counter unit)
and the library's kernels on the default workload; the summary scales each
kernel's counters by the copy's factors.  The JSON line reports that traffic
only while the kernel sources hash to the value recorded with it.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0   # MI355X HBM3E, vendor figure
HOST_LINK_PEAK_GBS = 64.0  # PCIe 5.0 x16, one direction: 32 GT/s x 16 lanes
LAYERS = 8
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "attention-decode-b8-16k_traffic.md")
CALIB_BYTES = 256 << 20   # bytes read (and written) by the calibration copy


def sources_sha256():
    """Hash of the kernel sources (the traffic figures are valid for these)."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "block_sparse_attention_nosa_amd", "csrc")
    for f in sorted(os.listdir(d)):
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_traffic(workload):
    """Bytes per attention launch from the committed counter summary, or None
    when it is missing, covers another workload or was taken on other kernel
    sources."""
    if workload != "decode-b8-16k":
        return None
    try:
        vals = {}
        with open(TRAFFIC_FILE) as fh:
            for line in fh:
                if line.startswith("- ") and ": " in line:
                    k, v = line[2:].strip().split(": ", 1)
                    vals[k] = v.strip("` ")
        if vals.get("sources_sha256") != sources_sha256():
            return None
        return int(vals["attention_traffic_bytes_per_launch"])
    except (OSError, KeyError, ValueError):
        return None


def algorithmic_bytes(w, lens, append: bool):
    """Bytes the method must move for one decode step (intermediates excluded):
    pooled keys read, K and V of the kept tokens, q in, out + lse written, and
    the pooled-key append (32 K rows read, one key written) when the current
    token completes a key.  Returns (step_bytes, attention_bytes)."""
    d, G, Hkv = w.head_dim, w.group, w.num_kv_heads
    wb = w.window // w.block_size
    step = attn = 0
    for L in lens:
        nc = (L - w.kernel) // w.stride + 1 if L >= w.kernel else 0
        nb = (L + w.block_size - 1) // w.block_size
        count = min(nb, w.topk + wb)
        tail = L - w.block_size * (nb - 1)
        toks = (count - 1) * w.block_size + tail if wb > 0 else count * w.block_size
        kv = toks * d * 2 * 2
        q_out = G * d * 2 + G * d * 4 + G * 4
        app = (w.kernel * d * 2 + d * 2) if append else 0
        step += Hkv * (nc * d * 2 + kv + q_out + app)
        attn += Hkv * (kv + q_out)
    return step, attn


def build_layers(w, nsteps, device="cuda"):
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth
    layers = []
    for li in range(LAYERS):
        wl = synth.Workload(**{**w.__dict__, "seed": w.seed + 7919 * li, "meta": {}})
        inp = synth.make_inputs(wl, device=device)
        pg = synth.to_paged(inp, wl, device=device)
        kv = nosa.paged_kv(pg["k_pool"], pg["v_pool"], pg["kc_pool"], pg["block_table"])
        p = nosa.params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel,
                        w.stride, w.topk, w.window, locality=w.locality)
        lens0 = [L - 1 for L in w.lens]
        nosa.nosa_compress_keys(p, kv, synth.cu_from_lens(lens0, device), None, w.batch,
                                max(lens0))
        layers.append(dict(inp=inp, pg=pg, kv=kv, p=p))
        torch.cuda.synchronize()
    return layers


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)  # multiple of 256, or <= 512
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--cpu-sample-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--locality", type=float, default=0.0,
                    help="share of the top-k budget forced to the blocks before the window")
    ap.add_argument("--prompt", type=int, default=0, metavar="TOKENS",
                    help="time the whole-prompt sparse prefill of one prompt of this length "
                         "(NOSA-1B head shape, top-k 64, window 1024) instead of a decode step")
    ap.add_argument("--chunk", type=int, default=4096,
                    help="queries per chunk of the whole-prompt prefill")
    ap.add_argument("--offload", action="store_true",
                    help="time the decode step over an offloaded KV cache (pages in pinned host "
                         "memory, a block cache in device memory) instead of device pools")
    ap.add_argument("--query-corr", type=float, default=0.9,
                    help="offload: correlation of each step's query with the previous step's "
                         "(q_t = c q_(t-1) + sqrt(1 - c^2) noise); 1 repeats the query")
    ap.add_argument("--cache-blocks", type=int, default=0,
                    help="offload: block-cache slots per (sequence, KV head); 0 = twice the "
                         "query-aware budget, at most 256")
    ap.add_argument("--front", type=int, default=0, metavar="HIDDEN",
                    help="time the attention layer's decode step from hidden states of this "
                         "width (QKV projection + rotary encoding + KV write, then the sparse "
                         "attention) instead of the step from ready queries")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run the calibration copy and the kernels once each for counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of --pmc-probe")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="table of a rocprofv3 --kernel-trace --stats csv run")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary)
    if args.trace_summary:
        return trace_summary(args.trace_summary)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth

    w = synth.config(args.config)
    if args.prompt:
        w = synth.Workload(lens=[args.prompt], q_lens=[args.prompt], topk=64, planted=0,
                           seed=1000 + args.prompt, name=f"prompt-prefill-{args.prompt}")
    if args.locality:
        w = synth.Workload(**{**w.__dict__, "locality": args.locality,
                              "name": f"{w.name}-locality{args.locality:g}"})
    if args.prompt:
        return prompt_main(w, args)
    if args.offload:
        return offload_main(w, args)
    if args.front:
        return front_main(w, args)
    if w.q_lens is not None:
        return prefill_main(w, args)
    nsteps = w.extra_tokens + 1
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_setup = time.time()
    layers = build_layers(w, nsteps)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens_at = [[L + t for L in w.lens] for t in range(nsteps)]
    cu_at = [synth.cu_from_lens(l, "cuda") for l in lens_at]
    maxL = max(lens_at[-1])
    p = layers[0]["p"]
    ws = torch.zeros(nosa.nosa_workspace_size(p, B, 1, maxL), dtype=torch.uint8, device=dev)
    out = torch.empty(B, Hq, d, device=dev)
    lse = torch.empty(B, Hq, device=dev)
    max_sel = w.topk + w.window // w.block_size
    sels = [torch.empty(B, 1, Hkv, max_sel, dtype=torch.int32, device=dev) for _ in layers]
    cnts = [torch.empty(B, 1, Hkv, dtype=torch.int32, device=dev) for _ in layers]
    qs = [l["inp"]["q"] for l in layers]
    stream = torch.cuda.current_stream()
    print(f"[bench] setup {time.time() - t_setup:.1f}s; workload {w.name}: B={B} heads={Hq}/{Hkv} "
          f"L={w.lens[0]}..{maxL} topk={w.topk} layers={LAYERS}", file=sys.stderr, flush=True)

    if args.pmc_probe:
        return pmc_probe(w, layers, lens_at, cu_at, maxL, ws, out, lse, sels, cnts, qs)

    def step(i):
        li = i % LAYERS
        t = (i // LAYERS) % nsteps
        L = layers[li]
        # launched on the current stream (the capture stream while capturing)
        nosa.nosa_decode_step(L["p"], L["kv"], qs[li], cu_at[t], B, maxL, out, lse, ws,
                              sel_idx=sels[li], sel_count=cnts[li])
        return t

    # The steps are captured in a HIP graph (the library launches on the
    # capture stream); replaying it removes host launch cost from the timing.
    chunk = args.steps if args.steps <= 512 or args.steps % 256 else 256
    reps = args.steps // chunk
    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph):
        ts = [step(args.warmup + i) for i in range(chunk)]
    graph.replay()
    torch.cuda.synchronize()
    # the replay must have run the steps: the outputs of the last captured
    # step are recomputed from a poisoned buffer
    out.fill_(float("nan"))
    graph.replay()
    torch.cuda.synchronize()
    assert torch.isfinite(out).all(), "graph replay did not run the decode steps"
    # ---- timed region: K whole decode steps
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    torch.cuda.synchronize()
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_total = e0.elapsed_time(e1)
    ms_step = ms_total / args.steps
    step_bytes = np.mean([algorithmic_bytes(w, lens_at[t], (lens_at[t][0] - w.kernel) % w.stride == 0)[0]
                          for t in ts])
    tokens_per_s = B / (ms_step * 1e-3)
    print(f"[bench] {args.steps} steps in {ms_total:.2f} ms -> {ms_step * 1e3:.2f} us/step, "
          f"{step_bytes / 1e6:.2f} MB/step, {step_bytes / (ms_step * 1e-3) / 1e9:.0f} GB/s",
          file=sys.stderr, flush=True)

    # ---- dominant kernel: the sparse attention over the kept pages (one
    # launch of nosa_sparse_attend = one kernel), timed alone with events on
    # its launch stream around a graph of 256 launches over the same layers
    # and positions
    na = 256
    attn_bytes = []
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for i in range(na):
            li = i % LAYERS
            t = (i // LAYERS) % nsteps
            L = layers[li]
            nosa.nosa_sparse_attend(L["p"], L["kv"], qs[li], None, cu_at[t], B, 1, maxL, sels[li],
                                    cnts[li], out, lse, ws)
            attn_bytes.append(algorithmic_bytes(w, lens_at[t], False)[1])
    ga.replay()
    torch.cuda.synchronize()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for _ in range(4):
        ga.replay()
    eb.record(stream)
    torch.cuda.synchronize()
    us_attn = ea.elapsed_time(eb) * 1e3 / (4 * na)
    attn_gbs = float(np.mean(attn_bytes)) / (us_attn * 1e-6) / 1e9

    # ---- CPU reference on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, layers[0], lens_at, args.cpu_sample_seconds)

    ctx_name = (f"{round((w.lens[0] - 1) / 1024)}K" if len(set(w.lens)) == 1 else "varlen")
    res = {
        "metric": f"sparse-attn decode tokens/s at {ctx_name} ctx, batch {B}; "
                  "achieved HBM GB/s vs peak",
        "value": round(tokens_per_s, 1),
        "unit": "tokens/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) K/V/q, planted blocks, permuted 64-token pages)",
        "config": {"workload": w.name, "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "head_dim": d, "context": w.lens[0] - 1, "decode_steps": nsteps,
                   "topk_blocks": w.topk, "window_tokens": w.window, "block": w.block_size,
                   "pool_kernel": w.kernel, "pool_stride": w.stride, "layer_caches": LAYERS,
                   "locality": w.locality},
        "step_hbm": {"algorithmic_bytes": int(step_bytes),
                     "achieved_gbs": round(step_bytes / (ms_step * 1e-3) / 1e9, 1),
                     "frac": round(step_bytes / (ms_step * 1e-3) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"kernel": "attend_kernel (nosa_sparse_attend: attention over the kept pages + merge)", "bound": "hbm",
                     "achieved": round(attn_gbs, 1), "peak": HBM_PEAK_GBS, "unit": "GB/s",
                     "frac": round(attn_gbs / HBM_PEAK_GBS, 4), "traffic": recorded_traffic(w.name),
                     "us_per_launch": round(us_attn, 3),
                     "algorithmic_bytes_per_launch": int(np.mean(attn_bytes))},
        "cpu_baseline": cpu,
    }
    print(json.dumps(res), flush=True)


MFMA_BF16_PEAK_TFLOPS = 2500.0  # MI355X dense bf16, vendor figure


def prefill_flops(w):
    """Algorithmic FLOPs of one chunk: q.Kc^T over the pooled keys each query
    sees (once), and q.K^T + P.V over the kept tokens each query sees
    (selection from the reference-equivalent GPU run is not needed: every
    kept block but the causal diagonal is full, so count min(nb, topk+16)
    blocks of 64 tokens capped at the query position)."""
    d = w.head_dim
    L, Lq = w.lens[0], w.q_lens[0]
    wb = w.window // w.block_size
    score = attn = 0
    for i in range(Lq):
        p = L - Lq + i
        nc = (p + 1 - w.kernel) // w.stride + 1 if p + 1 >= w.kernel else 0
        score += nc
        r = i // 64
        p_last = L - Lq + min(64 * r + 64, Lq) - 1
        nb = p_last // 64 + 1
        kept = min(nb, w.topk + wb)
        attn += (kept - 1) * 64 + (p - 64 * (nb - 1) + 1 if p >= 64 * (nb - 1) else 0)
    return 2.0 * d * score * w.num_q_heads, 4.0 * d * attn * w.num_q_heads


def prefill_main(w, args):
    """Chunked sparse prefill (not the headline metric): time the chain
    nosa_block_scores -> nosa_select_blocks -> nosa_sparse_attend on one
    chunk, graph-replayed, and report MFMA throughput."""
    import math
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth

    dev = torch.device("cuda", 0)
    inp = synth.make_inputs(w, device="cuda")
    pg = synth.to_paged(inp, w, device="cuda")
    kv = nosa.paged_kv(pg["k_pool"], pg["v_pool"], pg["kc_pool"], pg["block_table"])
    p = nosa.params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    B, maxL, maxLq = w.batch, max(w.lens), max(w.q_lens)
    cu_k = synth.cu_from_lens(w.lens, "cuda")
    cu_q = inp["cu_q"].cuda().to(torch.int32)
    nosa.nosa_compress_keys(p, kv, cu_k, None, B, maxL)
    mq = math.ceil(maxLq / 64)
    max_nb = math.ceil(maxL / 64)
    scores = torch.empty(B, mq, w.num_kv_heads, max_nb, device=dev)
    sel = torch.empty(B, mq, w.num_kv_heads, w.topk + w.window // 64, dtype=torch.int32, device=dev)
    cnt = torch.empty(B, mq, w.num_kv_heads, dtype=torch.int32, device=dev)
    out = torch.empty(inp["q"].shape[0], w.num_q_heads, w.head_dim, device=dev)
    lse = torch.empty(inp["q"].shape[0], w.num_q_heads, device=dev)
    ws = torch.zeros(nosa.nosa_workspace_size(p, B, maxLq, maxL), dtype=torch.uint8, device=dev)

    def chain():
        nosa.nosa_block_scores(p, kv, inp["q"], cu_q, cu_k, B, maxLq, maxL, scores, ws)
        nosa.nosa_select_blocks(p, scores, cu_q, cu_k, B, maxLq, maxL, sel, cnt)
        nosa.nosa_sparse_attend(p, kv, inp["q"], cu_q, cu_k, B, maxLq, maxL, sel, cnt, out, lse, ws)

    for _ in range(max(1, args.warmup // 16)):
        chain()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        chain()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // 64)
    e0, e1 = torch.cuda.Event(True), torch.cuda.Event(True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    fs, fa = prefill_flops(w)
    tf = (fs + fa) / (us * 1e-6) / 1e12
    res = {"metric": "sparse prefill chunk: MFMA TFLOP/s (algorithmic flops)", "value": round(tf, 2),
           "unit": "TFLOP/s", "n_gpus": 1, "steps": reps, "warmup": args.warmup,
           "ms_per_step": round(us / 1e3, 4), "higher_is_better": True, "scaling": "weak",
           "vs_baseline": None, "dtype": "bf16", "data": "synthetic (seeded bf16 N(0,1))",
           "config": {"workload": w.name, "queries": maxLq, "context": maxL,
                      "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "topk_blocks": w.topk},
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": None, "scoring_gflop": round(fs / 1e9, 2),
                        "attention_gflop": round(fa / 1e9, 2)}}
    print(json.dumps(res), flush=True)


def prompt_main(w, args):
    """Whole-prompt sparse prefill (not the headline metric): one
    nosa_prefill_sparse call over the prompt, chunk by chunk, graph-replayed;
    reports MFMA throughput over the algorithmic flops."""
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth

    dev = torch.device("cuda", 0)
    inp = synth.make_inputs(w, device="cuda")
    pg = synth.to_paged(inp, w, device="cuda")
    kv = nosa.paged_kv(pg["k_pool"], pg["v_pool"], pg["kc_pool"], pg["block_table"])
    p = nosa.params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    B, L = w.batch, max(w.lens)
    cu = synth.cu_from_lens(w.lens, "cuda")
    out = torch.empty(inp["q"].shape[0], w.num_q_heads, w.head_dim, device=dev)
    lse = torch.empty(inp["q"].shape[0], w.num_q_heads, device=dev)
    ws = torch.zeros(nosa.nosa_prefill_sparse_workspace_size(p, B, L, args.chunk),
                     dtype=torch.uint8, device=dev)

    def run():
        nosa.nosa_prefill_sparse(p, kv, inp["q"], cu, B, L, args.chunk, out, lse, ws)

    for _ in range(max(1, args.warmup // 16)):
        run()
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        run()
    g.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // 256)
    e0, e1 = torch.cuda.Event(True), torch.cuda.Event(True)
    e0.record()
    for _ in range(reps):
        g.replay()
    e1.record()
    torch.cuda.synchronize()
    us = e0.elapsed_time(e1) * 1e3 / reps
    fs, fa = prefill_flops(w)
    tf = (fs + fa) / (us * 1e-6) / 1e12
    res = {"metric": "whole-prompt sparse prefill: MFMA TFLOP/s (algorithmic flops)",
           "value": round(tf, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": reps,
           "warmup": args.warmup, "ms_per_step": round(us / 1e3, 4), "higher_is_better": True,
           "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
           "data": "synthetic (seeded bf16 N(0,1))",
           "config": {"workload": w.name, "prompt_tokens": L, "chunk": args.chunk,
                      "q_heads": w.num_q_heads, "kv_heads": w.num_kv_heads, "topk_blocks": w.topk,
                      "prompt_tokens_per_s": round(L * B / (us * 1e-6))},
           "roofline": {"bound": "mfma", "achieved": round(tf, 2), "peak": MFMA_BF16_PEAK_TFLOPS,
                        "unit": "TFLOP/s", "frac": round(tf / MFMA_BF16_PEAK_TFLOPS, 4),
                        "traffic": None, "scoring_gflop": round(fs / 1e9, 2),
                        "attention_gflop": round(fa / 1e9, 2)}}
    print(json.dumps(res), flush=True)


def front_main(w, args):
    """Decode steps of an attention layer from its hidden states (not the
    headline metric): per layer cache a packed QKV weight matrix (seeded
    N(0, 1/hidden)) and hidden states; a step is the front-end launch
    (projection, rotary encoding, K/V write into the pages) and the three
    launches of the sparse step.  The front-end kernel is also timed alone."""
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    hidden = args.front
    nsteps = w.extra_tokens + 1
    layers = build_layers(w, nsteps)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens_at = [[L + t for L in w.lens] for t in range(nsteps)]
    cu_at = [synth.cu_from_lens(l, "cuda") for l in lens_at]
    maxL = max(lens_at[-1])
    p = layers[0]["p"]
    rows = (Hq + 2 * Hkv) * d
    front = nosa.front_params(hidden, 10000.0)
    for li, L in enumerate(layers):
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed + 31337 * li)
        wt = (torch.randn(rows, hidden, generator=gen, device=dev) / hidden ** 0.5).to(torch.bfloat16)
        L["w"] = torch.empty_like(wt)
        nosa.nosa_pack_qkv_weights(p, hidden, wt, L["w"])
        L["x"] = torch.randn(B, hidden, generator=gen, device=dev).to(torch.bfloat16)
        del wt
    ws = torch.zeros(nosa.nosa_workspace_size(p, B, 1, maxL), dtype=torch.uint8, device=dev)
    q_out = torch.empty(B, Hq, d, dtype=torch.bfloat16, device=dev)
    out = torch.empty(B, Hq, d, device=dev)
    lse = torch.empty(B, Hq, device=dev)
    stream = torch.cuda.current_stream()

    def layer_step(i):
        li = i % LAYERS
        t = (i // LAYERS) % nsteps
        L = layers[li]
        nosa.nosa_layer_decode_step(p, front, L["kv"], L["x"], L["w"], cu_at[t], B, maxL, q_out,
                                    out, lse, ws)

    def front_only(i):
        li = i % LAYERS
        t = (i // LAYERS) % nsteps
        L = layers[li]
        nosa.nosa_qkv_rope_append(p, front, L["kv"], L["x"], L["w"], cu_at[t], B, maxL, q_out)

    def timed(fn, n):
        for i in range(16):
            fn(i)
        torch.cuda.synchronize()
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(n):
                fn(16 + i)
        g.replay()
        torch.cuda.synchronize()
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        for _ in range(4):
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        return e0.elapsed_time(e1) * 1e3 / (4 * n)

    n = 256
    us_layer = timed(layer_step, n)
    us_front = timed(front_only, n)
    w_bytes = rows * hidden * 2
    front_bytes = w_bytes + B * hidden * 2 + B * (Hq + 2 * Hkv) * d * 2
    front_gbs = front_bytes / (us_front * 1e-6) / 1e9
    attn_bytes = np.mean([algorithmic_bytes(w, lens_at[t], False)[0] for t in range(nsteps)])
    step_bytes = attn_bytes + front_bytes
    print(f"[bench] layer step from hidden {hidden}: {us_layer:.2f} us/step "
          f"({step_bytes / 1e6:.2f} MB: {step_bytes / (us_layer * 1e-6) / 1e9:.0f} GB/s); "
          f"front end alone {us_front:.2f} us ({front_gbs:.0f} GB/s)", file=sys.stderr, flush=True)
    res = {
        "metric": "attention-layer decode tokens/s from hidden states at 16K ctx, batch 8; "
                  "achieved HBM GB/s vs peak",
        "value": round(B / (us_layer * 1e-6), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": 4 * n, "warmup": 16, "ms_per_step": round(us_layer / 1e3, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) hidden states and K/V, N(0, 1/hidden) weights, "
                "planted blocks, permuted pages)",
        "config": {"workload": w.name + f"-from-hidden{hidden}", "batch": B, "q_heads": Hq,
                   "kv_heads": Hkv, "hidden": hidden, "context": w.lens[0] - 1,
                   "topk_blocks": w.topk, "window_tokens": w.window, "layer_caches": LAYERS},
        "step_hbm": {"algorithmic_bytes": int(step_bytes),
                     "achieved_gbs": round(step_bytes / (us_layer * 1e-6) / 1e9, 1),
                     "frac": round(step_bytes / (us_layer * 1e-6) / 1e9 / HBM_PEAK_GBS, 4)},
        "roofline": {"kernel": "front_kernel (QKV projection + rotary encoding + KV write)",
                     "bound": "hbm", "achieved": round(front_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(front_gbs / HBM_PEAK_GBS, 4), "traffic": None,
                     "us_per_launch": round(us_front, 3),
                     "algorithmic_bytes_per_launch": int(front_bytes)},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def offload_main(w, args):
    """Decode steps over an offloaded KV cache (not the headline metric): the
    K/V pages of every layer cache in pinned host memory, the recent pages in
    a device ring, a block cache per (sequence, KV head).  Each step's query
    is correlated with the previous one (--query-corr), so consecutive
    selections overlap the way decoding queries do; the step reads from host
    memory only the picks its cache misses."""
    import math
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth

    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_setup = time.time()
    nsteps = w.extra_tokens + 1
    layers = build_layers(w, nsteps)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens_at = [[L + t for L in w.lens] for t in range(nsteps)]
    cu_at = [synth.cu_from_lens(l, "cuda") for l in lens_at]
    maxL = max(lens_at[-1])
    p = layers[0]["p"]
    k_loc = math.floor(w.locality * w.topk + 0.5)
    wb = w.window // w.block_size + k_loc
    kq_budget = w.topk - k_loc
    cap = args.cache_blocks or min(256, 2 * kq_budget)
    # ring of recent pages: every block that is forced (or read by the key
    # append) at some step of the run, so the ring is written once
    lo = [max(0, (L + 63) // 64 - max(wb, 2)) for L in w.lens]
    hi = [(L + nsteps - 1 + 63) // 64 - 1 for L in w.lens]
    R = max(h - l + 1 for l, h in zip(lo, hi))
    rho = args.query_corr
    offs = []
    for li, L in enumerate(layers):
        pg = L["pg"]
        k_host = torch.empty(pg["k_pool"].shape, dtype=torch.bfloat16, pin_memory=True)
        v_host = torch.empty(pg["v_pool"].shape, dtype=torch.bfloat16, pin_memory=True)
        k_host.copy_(pg["k_pool"].cpu())
        v_host.copy_(pg["v_pool"].cpu())
        page = pg["k_pool"].shape[-1]
        k_ring = torch.zeros(B, R, Hkv, page, dtype=torch.bfloat16, device=dev)
        v_ring = torch.zeros_like(k_ring)
        for s in range(B):
            for b in range(lo[s], hi[s] + 1):
                pid = int(pg["block_table"][s, b])
                k_ring[s, b % R] = pg["k_pool"][pid]
                v_ring[s, b % R] = pg["v_pool"][pid]
        cache_k = torch.zeros(B, Hkv, cap, page, dtype=torch.bfloat16, device=dev)
        cache_v = torch.zeros_like(cache_k)
        cmap = torch.full((B, Hkv, cap), -1, dtype=torch.int32, device=dev)
        cused = torch.zeros((B, Hkv, cap), dtype=torch.int32, device=dev)
        okv = nosa.offload_kv(k_host, v_host, pg["kc_pool"], pg["block_table"], k_ring, v_ring,
                              cache_k, cache_v, cmap, cused)
        gen = torch.Generator(device=dev)
        gen.manual_seed(w.seed + 104729 * li)
        qf = L["inp"]["q"].float()
        qs = []
        for t in range(nsteps):
            if t:
                qf = rho * qf + math.sqrt(max(0.0, 1 - rho * rho)) * torch.randn(
                    qf.shape, generator=gen, device=dev)
            qs.append(qf.to(torch.bfloat16))
        # the device pools are not used any more: only the host copies are read
        del pg["k_pool"], pg["v_pool"], L["kv"]
        offs.append(dict(okv=okv, qs=qs, keep=(k_host, v_host, k_ring, v_ring, cache_k, cache_v,
                                                cmap, cused)))
    torch.cuda.empty_cache()
    ws = torch.zeros(nosa.nosa_offload_workspace_size(p, B, maxL, cap), dtype=torch.uint8,
                     device=dev)
    out = torch.empty(B, Hq, d, device=dev)
    lse = torch.empty(B, Hq, device=dev)
    chunk = LAYERS * nsteps  # one graph runs every step of every layer cache once
    fetch = torch.zeros(chunk, B, Hkv, dtype=torch.int32, device=dev)
    stream = torch.cuda.current_stream()
    print(f"[bench] setup {time.time() - t_setup:.1f}s; offloaded {w.name}: ring {R} blocks, "
          f"cache {cap} blocks, query correlation {rho}", file=sys.stderr, flush=True)

    def step(i):
        li = i % LAYERS
        t = (i // LAYERS) % nsteps
        o = offs[li]
        nosa.nosa_offload_decode_step(p, o["okv"], o["qs"][t], cu_at[t], B, maxL, out, lse, ws,
                                      fetch_count=fetch[i % chunk])
        return t

    for i in range(args.warmup):
        step(i)
    torch.cuda.synchronize()
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.graph(graph, capture_error_mode="relaxed"):
        ts = [step(args.warmup + i) for i in range(chunk)]
    graph.replay()
    torch.cuda.synchronize()
    reps = max(1, args.steps // chunk)
    e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    e0.record(stream)
    for _ in range(reps):
        graph.replay()
    e1.record(stream)
    torch.cuda.synchronize()
    ms_step = e0.elapsed_time(e1) / (reps * chunk)
    fetched = fetch.double().sum().item() / chunk  # blocks per step, last replay
    picks = np.mean([sum(min(kq_budget, max(0, (L + 63) // 64 - wb)) for L in lens_at[t]) * Hkv
                     for t in ts])
    blk_bytes = 2 * w.block_size * d * 2  # K and V of one block of one KV head
    host_gbs = fetched * blk_bytes / (ms_step * 1e-3) / 1e9
    # the link itself: one large pinned-host to device copy
    src = torch.empty(256 << 20, dtype=torch.uint8, pin_memory=True)
    dst = torch.empty(256 << 20, dtype=torch.uint8, device=dev)
    dst.copy_(src, non_blocking=True)
    torch.cuda.synchronize()
    c0, c1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    c0.record(stream)
    for _ in range(4):
        dst.copy_(src, non_blocking=True)
    c1.record(stream)
    torch.cuda.synchronize()
    copy_gbs = 4 * (256 << 20) / (c0.elapsed_time(c1) * 1e-3) / 1e9
    print(f"[bench] {reps * chunk} offloaded steps: {ms_step * 1e3:.1f} us/step, "
          f"{fetched:.1f} of {picks:.1f} picks read from host per step, {host_gbs:.1f} GB/s "
          f"(host-to-device copy {copy_gbs:.1f} GB/s)", file=sys.stderr, flush=True)
    res = {
        "metric": "offloaded-KV sparse-attn decode tokens/s, batch 8, 16K ctx; host-link GB/s "
                  "of the fetched blocks",
        "value": round(B / (ms_step * 1e-3), 1), "unit": "tokens/s", "n_gpus": 1,
        "steps": reps * chunk, "warmup": args.warmup, "ms_per_step": round(ms_step, 5),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic (seeded bf16 N(0,1) K/V, planted blocks, permuted pages; queries "
                "correlated from step to step)",
        "config": {"workload": w.name + "-offloaded", "batch": B, "q_heads": Hq, "kv_heads": Hkv,
                   "context": w.lens[0] - 1, "decode_steps": nsteps, "topk_blocks": w.topk,
                   "window_tokens": w.window, "locality": w.locality, "query_corr": rho,
                   "cache_blocks": cap, "recent_blocks": R, "layer_caches": LAYERS,
                   "picks_per_step": round(float(picks), 1),
                   "fetched_blocks_per_step": round(fetched, 2),
                   "fetched_fraction": round(fetched / picks, 4) if picks else 0.0},
        "roofline": {"kernel": "top_kernel (offloaded: picks missing from the cache read from "
                               "host memory)", "bound": "host-link",
                     "achieved": round(host_gbs, 2), "peak": HOST_LINK_PEAK_GBS, "unit": "GB/s",
                     "frac": round(host_gbs / HOST_LINK_PEAK_GBS, 4), "traffic": None,
                     "measured_copy_gbs": round(copy_gbs, 2)},
        "cpu_baseline": None,
    }
    print(json.dumps(res), flush=True)


def pmc_probe(w, layers, lens_at, cu_at, maxL, ws, out, lse, sels, cnts, qs):
    """One pass of every kernel for counter collection: the calibration copy
    (CALIB_BYTES read, CALIB_BYTES written), then per layer one decode step
    and one stand-alone attention over its selection."""
    import torch
    from block_sparse_attention_nosa_amd import nosa
    a = torch.ones(CALIB_BYTES // 4, dtype=torch.int32, device="cuda")
    b = torch.empty_like(a)
    for _ in range(2):
        torch.bitwise_not(a, out=b)  # a kernel used nowhere else: reads a, writes b
    torch.cuda.synchronize()
    B = w.batch
    for li, L in enumerate(layers):
        nosa.nosa_decode_step(L["p"], L["kv"], qs[li], cu_at[0], B, maxL, out, lse, ws,
                              sel_idx=sels[li], sel_count=cnts[li])
        nosa.nosa_sparse_attend(L["p"], L["kv"], qs[li], None, cu_at[0], B, 1, maxL, sels[li],
                                cnts[li], out, lse, ws)
    torch.cuda.synchronize()
    attn = algorithmic_bytes(w, lens_at[0], False)[1]
    print(f"[pmc-probe] done; attention algorithmic bytes per launch {attn}", file=sys.stderr)


def _pmc_rows(d, counter):
    """(kernel name, value) per dispatch of one counter from a rocprofv3 csv run."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*counter_collection.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no counter_collection.csv under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            for r in csv.DictReader(fh):
                if r.get("Counter_Name") == counter:
                    rows.append((r["Kernel_Name"], float(r["Counter_Value"])))
    return rows


def pmc_summary(fetch_dir, write_dir):
    """Markdown summary of FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel,
    scaled to bytes by the calibration copy, and the attention's traffic per
    launch (its attention kernel plus its merge)."""
    import numpy as np
    from block_sparse_attention_nosa_amd import synth
    w = synth.config(2)
    attn_alg = algorithmic_bytes(w, w.lens, False)[1]
    per = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        for name, v in _pmc_rows(d, counter):
            per.setdefault(name, {}).setdefault(counter, []).append(v)
    calib = [n for n in per if "bitwise_not" in n.lower() or "BitwiseNot" in n]
    if not calib:
        raise SystemExit("calibration copy kernel not found")
    c = per[calib[0]]
    f_fetch = CALIB_BYTES / (np.median(c["FETCH_SIZE"]) * 1024.0)
    f_write = CALIB_BYTES / (np.median(c["WRITE_SIZE"]) * 1024.0)
    lines = ["# HBM traffic of the decode-b8-16k kernels (rocprofv3 counters)", "",
             "Commands (from the repository root):", "",
             "    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o run --output-format csv -- python3 bench.py --pmc-probe",
             "    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o run --output-format csv -- python3 bench.py --pmc-probe",
             "    python3 bench.py --pmc-summary DIR_F DIR_W", "",
             f"Calibration: a plain copy reading and writing {CALIB_BYTES >> 20} MiB; "
             f"bytes per counter KiB: fetch {f_fetch * 1024:.1f}, write {f_write * 1024:.1f} "
             f"(factors {f_fetch:.3f} / {f_write:.3f} of the nominal 1024).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB |",
             "|---|---:|---:|---:|---:|---:|"]
    traffic = {}
    for name in sorted(per):
        v = per[name]
        if "FETCH_SIZE" not in v or "WRITE_SIZE" not in v:
            continue
        if not ("nosa::" in name or name in calib):
            continue
        fk, wk = float(np.mean(v["FETCH_SIZE"])), float(np.mean(v["WRITE_SIZE"]))
        fb, wb = fk * 1024 * f_fetch, wk * 1024 * f_write
        traffic[name] = fb + wb
        lines.append(f"| `{name[:90]}` | {len(v['FETCH_SIZE'])} | {fk:.0f} | {wk:.0f} | "
                     f"{fb / 1e6:.2f} | {wb / 1e6:.2f} |")
    attn_k = [n for n in traffic if "attend_kernel<" in n]
    merge_k = [n for n in traffic if "merge_kernel" in n]
    if not attn_k or not merge_k:
        raise SystemExit("attention kernels not found")
    attn_t = traffic[attn_k[0]] + traffic[merge_k[0]]
    lines += ["", "The attention launch (nosa_sparse_attend) is its attention kernel plus its merge "
              "kernel; the merge row averages the dispatches of both entry points.", "",
              f"- attention_traffic_bytes_per_launch: {int(attn_t)}",
              f"- attention_algorithmic_bytes_per_launch: {int(attn_alg)}",
              f"- traffic_over_algorithmic: {attn_t / attn_alg:.3f}",
              f"- sources_sha256: {sources_sha256()}"]
    print("\n".join(lines))


def trace_summary(d):
    """Markdown rows (library kernels) of a rocprofv3 kernel_stats.csv."""
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", "*kernel_stats.csv"), recursive=True)
    if not files:
        raise SystemExit(f"no kernel_stats.csv under {d}")
    print("| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |")
    print("|---|---:|---:|---:|---:|---:|")
    with open(files[0]) as fh:
        for r in csv.DictReader(fh):
            if "nosa::" not in r["Name"]:
                continue
            name = r["Name"].split("(")[0] if r["Name"].startswith("nosa::") else r["Name"].split("(nosa")[0]
            print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
                  f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
                  f"{float(r['Percentage']):.1f}% |")


def cpu_baseline(w, layer, lens_at, budget_s):
    """The CPU reference as it stands, on host copies of layer 0: whole decode
    steps (pooling, scoring, selection, attention) for the full batch, repeated
    until about `budget_s` seconds of work."""
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import synth
    from oracle import oracle as ora

    inp = layer["inp"]
    host = dict(k=inp["k"].cpu(), v=inp["v"].cpu(), cu_k_store=inp["cu_k_store"].cpu())
    q = synth.bits(inp["q"])
    op = ora.Params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    n, t0 = 0, time.time()
    while True:
        k, v, cu = synth.packed_live(host, w, n % len(lens_at))
        ora.forward(op, q, None, synth.bits(k), synth.bits(v), cu.numpy())
        n += 1
        if time.time() - t0 >= budget_s or n >= 64:
            break
    dt = time.time() - t0
    return {"value": round(w.batch * n / dt, 2), "unit": "tokens/s", "cores": ora.num_threads(),
            "kind": "oracle",
            "sample": f"{n} whole decode steps of {w.name} (batch {w.batch}, layer 0, positions "
                      f"0..{n - 1}) on the host, fp64 reference with OpenMP over (sequence, head)"}


if __name__ == "__main__":
    main()
