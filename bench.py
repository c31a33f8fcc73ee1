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
time), the roofline of the timed step (its algorithmic bytes over the step
time; the dominant kernel, top_kernel, named with its share from the
committed kernel trace), the stand-alone attention entry point timed with
HIP events on its own stream as a secondary figure, and the CPU reference's
throughput on a bounded sample of the same workload.

Traffic counters (kept out of the timed run):
    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o run --output-format csv -- python bench.py --pmc-probe
    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o run --output-format csv -- python bench.py --pmc-probe
    python bench.py --pmc-summary DIR_F DIR_W > profiles/decode-b8-16k_traffic.md
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
TRAFFIC_FILE = os.path.join(ROOT, "profiles", "decode-b8-16k_traffic.md")
TRACE_FILE = os.path.join(ROOT, "profiles", "decode-b8-16k_kernel_trace.md")
CALIB_BYTES = 256 << 20   # bytes read (and written) by the calibration copy


def sources_sha256():
    """Hash of the NOSA library's sources (the traffic figures are valid for
    these; the machine probes, a library of their own, are not hashed)."""
    import hashlib
    h = hashlib.sha256()
    d = os.path.join(ROOT, "block_sparse_attention_nosa_amd", "csrc")
    for f in sorted(os.listdir(d)):
        if f.startswith("probe_"):
            continue
        with open(os.path.join(d, f), "rb") as fh:
            h.update(f.encode() + b"\0" + fh.read())
    return h.hexdigest()


def recorded_traffic(workload, kind):
    """HBM bytes per decode step (kind "step": its three kernels) or per
    stand-alone attention launch (kind "attention") from the committed counter
    summary, or None when it is missing, covers another workload or was taken
    on other kernel sources."""
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
        return int(vals[f"{kind}_traffic_bytes"])
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


def build_layers(w, nsteps, device="cuda", nlayers=LAYERS, full_kc=False):
    """nlayers independent caches of workload w (seeds differ).  Pooled keys
    are built for the tokens before the first decode position, or with
    full_kc for every stored token (then any decode position can run in any
    order: a step reads only the keys of its own tokens and re-appends the
    key its token completes, bit for bit the same)."""
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth
    layers = []
    for li in range(nlayers):
        wl = synth.Workload(**{**w.__dict__, "seed": w.seed + 7919 * li, "meta": {}})
        inp = synth.make_inputs(wl, device=device)
        pg = synth.to_paged(inp, wl, device=device)
        kv = nosa.paged_kv(pg["k_pool"], pg["v_pool"], pg["kc_pool"], pg["block_table"])
        p = nosa.params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel,
                        w.stride, w.topk, w.window, locality=w.locality)
        lens0 = [L + w.extra_tokens if full_kc else L - 1 for L in w.lens]
        nosa.nosa_compress_keys(p, kv, synth.cu_from_lens(lens0, device), None, w.batch,
                                max(lens0))
        layers.append(dict(inp=inp, pg=pg, kv=kv, p=p))
        torch.cuda.synchronize()
    return layers


def step_positions(npos, steps, replays):
    """Decode position of every step of `replays` timed replays of `steps`
    steps: spread evenly, in order, over all npos positions (each position at
    least once when replays * steps >= npos), so window shifts (a new block)
    and pooled-key appends fall inside the timed region whatever `steps` is."""
    total = steps * replays
    return [g * npos // total for g in range(total)]


def time_decode(w, steps, warmup, min_replays=5, nlayers=LAYERS, check=True, static=False):
    """Whole decode steps of workload w (one nosa_decode_step call on the
    batch each): `warmup` eager steps, then replays of `steps` graph-captured
    steps each, timed one replay at a time with events on the launch stream
    between device synchronisations.  Step g of the run uses layer cache
    g % nlayers at position step_positions(...)[g].  Returns the median and
    every replay's time per step, the mean algorithmic bytes per step and the
    objects the caller reuses."""
    import math
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth
    nsteps = w.extra_tokens + 1
    layers = build_layers(w, nsteps, nlayers=nlayers, full_kc=True)
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    lens_at = [[L + t for L in w.lens] for t in range(nsteps)]
    cu_at = [synth.cu_from_lens(l, "cuda") for l in lens_at]
    maxL = max(lens_at[-1])
    p = layers[0]["p"]
    ws = torch.zeros(nosa.nosa_workspace_size(p, B, 1, maxL), dtype=torch.uint8, device="cuda")
    out = torch.empty(B, Hq, d, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")
    max_sel = w.topk + w.window // w.block_size
    sels = [torch.empty(B, 1, Hkv, max_sel, dtype=torch.int32, device="cuda") for _ in layers]
    cnts = [torch.empty(B, 1, Hkv, dtype=torch.int32, device="cuda") for _ in layers]
    qs = [l["inp"]["q"] for l in layers]
    replays = max(min_replays, math.ceil(nsteps / max(1, steps)))
    pos = step_positions(nsteps, steps, replays)

    def step(g, t):
        L = layers[g % nlayers]
        if static:
            nosa.nosa_decode_step_static(L["p"], L["kv"], qs[g % nlayers], cu_at[t], B, maxL,
                                         out, lse, sel_idx=sels[g % nlayers],
                                         sel_count=cnts[g % nlayers])
        else:
            nosa.nosa_decode_step(L["p"], L["kv"], qs[g % nlayers], cu_at[t], B, maxL, out, lse,
                                  ws, sel_idx=sels[g % nlayers], sel_count=cnts[g % nlayers])

    for i in range(warmup):
        step(i, pos[i % len(pos)])
    torch.cuda.synchronize()
    # one replay = graphs of at most 256 steps each, replayed back to back
    graphs = []
    for r in range(replays):
        gs = []
        for c0 in range(0, steps, 256):
            g = torch.cuda.CUDAGraph()
            with torch.cuda.graph(g):
                for i in range(c0, min(steps, c0 + 256)):
                    step(r * steps + i, pos[r * steps + i])
            gs.append(g)
        graphs.append(gs)
    stream = torch.cuda.current_stream()
    if check:  # the replays run the steps: the last step's output is rebuilt from poison
        out.fill_(float("nan"))
        for g in graphs[0]:
            g.replay()
        torch.cuda.synchronize()
        assert torch.isfinite(out).all(), "graph replay did not run the decode steps"
    times = []
    for r in range(replays):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        torch.cuda.synchronize()
        e0.record(stream)
        for g in graphs[r]:
            g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        times.append(e0.elapsed_time(e1) / steps)
    step_bytes = float(np.mean([algorithmic_bytes(w, lens_at[t], (lens_at[t][0] - w.kernel) % w.stride == 0)[0]
                                for t in pos]))
    appends = sum(1 for t in pos if (lens_at[t][0] - w.kernel) % w.stride == 0)
    shifts = sum(1 for t in pos if (lens_at[t][0] - 1) % w.block_size == 0)
    del graphs
    return dict(ms_per_step=float(np.median(times)), replay_ms=times, step_bytes=step_bytes,
                replays=replays, positions=len(set(pos)), append_steps=appends,
                shift_steps=shifts, layers=layers, lens_at=lens_at, cu_at=cu_at, maxL=maxL, ws=ws,
                out=out, lse=lse, sels=sels, cnts=cnts, qs=qs, nsteps=nsteps)


def copy_bandwidth(nbytes=2 << 30, reps=5):
    """A plain device-to-device copy of nbytes (read + write), median of
    reps: GB/s of bytes moved (2 nbytes per copy)."""
    import numpy as np
    import torch
    a = torch.empty(nbytes // 2, dtype=torch.bfloat16, device="cuda").fill_(1.0)
    b = torch.empty_like(a)
    b.copy_(a)
    torch.cuda.synchronize()
    ts = []
    for _ in range(reps):
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record()
        b.copy_(a)
        e1.record()
        torch.cuda.synchronize()
        ts.append(e0.elapsed_time(e1))
    del a, b
    torch.cuda.empty_cache()
    return 2 * nbytes / (float(np.median(ts)) * 1e-3) / 1e9


def device_record():
    """The device's own figures as the HIP runtime reports them (hipDeviceProp
    through torch), recorded beside the vendor peaks the fractions use."""
    import torch
    pr = torch.cuda.get_device_properties(0)
    rec = {"name": pr.name, "arch": getattr(pr, "gcnArchName", None),
           "compute_units": pr.multi_processor_count,
           "hbm_bytes": int(pr.total_memory),
           "l2_bytes": getattr(pr, "L2_cache_size", None),
           "lds_bytes_per_workgroup": getattr(pr, "shared_memory_per_block", None),
           "wave_size": getattr(pr, "warp_size", None)}
    return {k: v for k, v in rec.items() if v is not None}


def trace_average_us(path, kernel_prefix):
    """Average duration of a kernel in a committed kernel-trace summary, if
    the summary was taken on the current kernel sources."""
    try:
        txt = open(path).read()
    except OSError:
        return None
    if f"sources_sha256: {sources_sha256()}" not in txt:
        return None
    for line in txt.splitlines():
        if line.startswith("| `") and kernel_prefix in line:
            cells = [c.strip() for c in line.strip("|").split("|")]
            return float(cells[2])
    return None


def main():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=2048)
    ap.add_argument("--warmup", type=int, default=64)
    ap.add_argument("--config", type=int, default=2)
    ap.add_argument("--replays", type=int, default=5,
                    help="timed replays of --steps steps (at least 5; more when needed to cover "
                         "every decode position); the line reports their median")
    ap.add_argument("--cpu-sample-seconds", type=float, default=15.0)
    ap.add_argument("--no-cpu", action="store_true")
    ap.add_argument("--no-extra", action="store_true",
                    help="skip the other decode workloads (varlen batch 32, 64K batch 16) that "
                         "the default run also times")
    ap.add_argument("--static", action="store_true",
                    help="time nosa_decode_step_static (no workspace) instead of nosa_decode_step")
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
    ap.add_argument("--ceiling", action="store_true",
                    help="measure the chip's read ceilings instead: a 2 GiB stream read, a 2 GiB "
                         "copy and a gather of 32 KB pages in random order")
    ap.add_argument("--pmc-probe", action="store_true",
                    help="run the calibration copy and the kernels once each for counters")
    ap.add_argument("--pmc-summary", nargs=2, metavar=("FETCH_DIR", "WRITE_DIR"),
                    help="summarise two rocprofv3 --pmc runs of --pmc-probe")
    ap.add_argument("--chip-probes", action="store_true",
                    help="measure the chip costs the design rests on (instruction-mix overlap, LDS "
                         "bandwidth, in-launch hand-off, dependent-load latency)")
    ap.add_argument("--counter-table", nargs="+", metavar="DIR",
                    help="print a markdown table of the library kernels' counters from "
                         "rocprofv3 --pmc output directories")
    ap.add_argument("--timeline", action="store_true",
                    help="per-phase timeline of the decode step from the wall-clock stamps of "
                         "libnosa_timeline.so (the same kernels with stamps)")
    ap.add_argument("--trace-summary", metavar="DIR",
                    help="table of a rocprofv3 --kernel-trace --stats csv run")
    args = ap.parse_args()
    if args.pmc_summary:
        return pmc_summary(*args.pmc_summary)
    if args.trace_summary:
        return trace_summary(args.trace_summary)
    if args.counter_table:
        return counter_table(args.counter_table)
    if args.gpus != 1 or int(os.environ.get("WORLD_SIZE", "1")) > 1:
        print("bench.py measures one GPU only: the library has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)

    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import nosa, synth

    if args.chip_probes:
        return chip_probes_main(args)
    if args.timeline:
        w = synth.config(args.config)
        if w.q_lens is not None and max(w.q_lens) > 1:
            return timeline_prefill_main(w, args)
        return timeline_main(w, args)
    if args.ceiling:
        return ceiling_main(args)
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
    dev = torch.device("cuda", 0)
    torch.cuda.set_device(dev)
    t_setup = time.time()
    B, Hq, Hkv, d = w.batch, w.num_q_heads, w.num_kv_heads, w.head_dim
    if args.pmc_probe:
        nsteps = w.extra_tokens + 1
        layers = build_layers(w, nsteps)
        lens_at = [[L + t for L in w.lens] for t in range(nsteps)]
        cu_at = [synth.cu_from_lens(l, "cuda") for l in lens_at]
        maxL = max(lens_at[-1])
        ws = torch.zeros(nosa.nosa_workspace_size(layers[0]["p"], B, 1, maxL), dtype=torch.uint8,
                         device=dev)
        out, lse = torch.empty(B, Hq, d, device=dev), torch.empty(B, Hq, device=dev)
        max_sel = w.topk + w.window // w.block_size
        sels = [torch.empty(B, 1, Hkv, max_sel, dtype=torch.int32, device=dev) for _ in layers]
        cnts = [torch.empty(B, 1, Hkv, dtype=torch.int32, device=dev) for _ in layers]
        qs = [l["inp"]["q"] for l in layers]
        return pmc_probe(w, layers, lens_at, cu_at, maxL, ws, out, lse, sels, cnts, qs)

    # ---- timed region: K whole decode steps per replay, median of the replays
    r = time_decode(w, args.steps, args.warmup, max(5, args.replays), static=args.static)
    ms_step, step_bytes = r["ms_per_step"], r["step_bytes"]
    tokens_per_s = B / (ms_step * 1e-3)
    step_gbs = step_bytes / (ms_step * 1e-3) / 1e9
    print(f"[bench] setup+timing {time.time() - t_setup:.1f}s; workload {w.name}: B={B} "
          f"heads={Hq}/{Hkv} L={w.lens[0]}..{r['maxL']} topk={w.topk} layers={LAYERS}; "
          f"{r['replays']} replays of {args.steps} steps over {r['positions']} positions "
          f"({r['append_steps']} appending, {r['shift_steps']} starting a block): "
          f"median {ms_step * 1e3:.2f} us/step (replays "
          f"{', '.join(f'{x * 1e3:.2f}' for x in r['replay_ms'])}), "
          f"{step_bytes / 1e6:.2f} MB/step, {step_gbs:.0f} GB/s", file=sys.stderr, flush=True)
    layers, lens_at, cu_at, maxL = r["layers"], r["lens_at"], r["cu_at"], r["maxL"]
    nsteps = r["nsteps"]
    timing = {"replays": r["replays"], "steps_per_replay": args.steps, "statistic": "median",
              "replay_us_per_step": [round(x * 1e3, 3) for x in r["replay_ms"]],
              "decode_positions": r["positions"], "appending_steps": r["append_steps"],
              "block_starting_steps": r["shift_steps"]}

    # ---- the stand-alone attention (nosa_sparse_attend: attend_kernel +
    # merge) on the steps' selections, a 256-launch graph timed with events
    na = 256
    attn_bytes = []
    ga = torch.cuda.CUDAGraph()
    with torch.cuda.graph(ga):
        for i in range(na):
            li = i % LAYERS
            t = (i // LAYERS) % nsteps
            L = layers[li]
            nosa.nosa_sparse_attend(L["p"], L["kv"], r["qs"][li], None, cu_at[t], B, 1, maxL,
                                    r["sels"][li], r["cnts"][li], r["out"], r["lse"], r["ws"])
            attn_bytes.append(algorithmic_bytes(w, lens_at[t], False)[1])
    ga.replay()
    torch.cuda.synchronize()
    stream = torch.cuda.current_stream()
    ea, eb = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    ea.record(stream)
    for _ in range(4):
        ga.replay()
    eb.record(stream)
    torch.cuda.synchronize()
    us_attn = ea.elapsed_time(eb) * 1e3 / (4 * na)
    attn_gbs = float(np.mean(attn_bytes)) / (us_attn * 1e-6) / 1e9
    del ga, layers, r
    torch.cuda.empty_cache()

    # ---- a plain 2 GiB device-to-device copy on the same box
    copy_gbs = copy_bandwidth()

    # ---- the other decode workloads, timed in the same run (not the headline)
    extra = {}
    if not args.no_extra and args.config == 2 and not args.locality and not args.static:
        for n, nl in ((3, 4), (4, 2)):
            wx = synth.config(n)
            wx = synth.Workload(**{**wx.__dict__, "extra_tokens": 15})
            rx = time_decode(wx, 64, 8, 5, nlayers=nl)
            gbs = rx["step_bytes"] / (rx["ms_per_step"] * 1e-3) / 1e9
            extra[wx.name] = {"us_per_step": round(rx["ms_per_step"] * 1e3, 2),
                              "tokens_per_s": round(wx.batch / (rx["ms_per_step"] * 1e-3), 1),
                              "algorithmic_bytes": int(rx["step_bytes"]),
                              "achieved_gbs": round(gbs, 1),
                              "frac": round(gbs / HBM_PEAK_GBS, 4),
                              "replays": rx["replays"], "steps_per_replay": 64,
                              "layer_caches": nl, "decode_positions": 16}
            print(f"[bench] {wx.name}: {rx['ms_per_step'] * 1e3:.2f} us/step, "
                  f"{gbs:.0f} GB/s ({gbs / HBM_PEAK_GBS:.3f})", file=sys.stderr, flush=True)
            del rx
            torch.cuda.empty_cache()

    # ---- CPU reference on a bounded sample of the same workload
    cpu = None
    if not args.no_cpu:
        cpu = cpu_baseline(w, args.cpu_sample_seconds)

    top_us = trace_average_us(TRACE_FILE, "top_kernel<") if w.name == "decode-b8-16k" else None
    top_bytes = algorithmic_bytes(w, w.lens, False)[1]
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
                   "locality": w.locality, "entry_point": "nosa_decode_step_static"
                   if args.static else "nosa_decode_step"},
        "timing": timing,
        "roofline": {"kernel": "nosa_decode_step: score_kernel + top_kernel + merge_kernel "
                               "(the whole timed step)",
                     "bound": "hbm", "achieved": round(step_gbs, 1), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(step_gbs / HBM_PEAK_GBS, 4),
                     "traffic": recorded_traffic(w.name, "step"),
                     "algorithmic_bytes_per_step": int(step_bytes),
                     "frac_of_measured_copy": round(step_gbs / copy_gbs, 4),
                     "measured_copy_gbs": round(copy_gbs, 1),
                     "dominant_kernel": None if top_us is None else {
                         "name": "top_kernel (selection + window and top-k pages)",
                         "us_per_launch": top_us, "algorithmic_bytes": int(top_bytes),
                         "achieved": round(top_bytes / (top_us * 1e-6) / 1e9, 1),
                         "frac": round(top_bytes / (top_us * 1e-6) / 1e9 / HBM_PEAK_GBS, 4),
                         "source": os.path.relpath(TRACE_FILE, ROOT)}},
        "attend_only": {"kernel": "nosa_sparse_attend (attend_kernel + merge_kernel)",
                        "us_per_launch": round(us_attn, 3),
                        "algorithmic_bytes_per_launch": int(np.mean(attn_bytes)),
                        "achieved": round(attn_gbs, 1),
                        "frac": round(attn_gbs / HBM_PEAK_GBS, 4),
                        "traffic": recorded_traffic(w.name, "attention")},
        "other_workloads": extra or None,
        "cpu_baseline": cpu,
        "device": device_record(),
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
        torch.cuda.synchronize()
        nosa.nosa_sparse_attend(L["p"], L["kv"], qs[li], None, cu_at[0], B, 1, maxL, sels[li],
                                cnts[li], out, lse, ws)
        torch.cuda.synchronize()
    step, attn = algorithmic_bytes(w, lens_at[0], False)
    print(f"[pmc-probe] done; algorithmic bytes per step {step}, per attention launch {attn}",
          file=sys.stderr)


def _csv_rows(d, pattern):
    import csv
    import glob
    files = glob.glob(os.path.join(d, "**", pattern), recursive=True)
    if not files:
        raise SystemExit(f"no {pattern} under {d}")
    rows = []
    for f in files:
        with open(f) as fh:
            rows.extend(csv.DictReader(fh))
    return rows


def _pmc_rows(d, counter):
    """(dispatch id, kernel name, value) per dispatch of one counter from a
    rocprofv3 csv run, in dispatch order."""
    rows = [(int(r.get("Dispatch_Id", 0) or 0), r["Kernel_Name"], float(r["Counter_Value"]))
            for r in _csv_rows(d, "*counter_collection.csv") if r.get("Counter_Name") == counter]
    return sorted(rows)


def pmc_summary(fetch_dir, write_dir):
    """Markdown summary of FETCH_SIZE / WRITE_SIZE (KiB per dispatch) per kernel,
    scaled to bytes by the calibration copy: the traffic of one decode step
    (its scoring, top and merge dispatches) and of one stand-alone attention
    launch (its attention and merge dispatches)."""
    import numpy as np
    from block_sparse_attention_nosa_amd import synth
    w = synth.config(2)
    step_alg, attn_alg = algorithmic_bytes(w, w.lens, False)
    per = {}   # role -> counter -> values
    names = {}
    for counter, d in (("FETCH_SIZE", fetch_dir), ("WRITE_SIZE", write_dir)):
        prev = None
        for _, name, v in _pmc_rows(d, counter):
            if "bitwise_not" in name.lower() or "BitwiseNot" in name:
                role = "calibration copy"
            elif "nosa::" not in name:
                prev = None
                continue
            elif "merge_kernel" in name:
                role = "merge_kernel (decode step)" if prev == "top" else "merge_kernel (attention)"
            else:
                role = name.split("(")[0].replace("void ", "")
                prev = "top" if "top_kernel" in name else ("attend" if "attend_kernel" in name else prev)
            names[role] = name
            per.setdefault(role, {}).setdefault(counter, []).append(v)
    c = per.get("calibration copy")
    if not c:
        raise SystemExit("calibration copy kernel not found")
    f_fetch = CALIB_BYTES / (np.median(c["FETCH_SIZE"]) * 1024.0)
    f_write = CALIB_BYTES / (np.median(c["WRITE_SIZE"]) * 1024.0)
    lines = ["# HBM traffic of the decode-b8-16k kernels (rocprofv3 counters)", "",
             "Commands (from the repository root):", "",
             "    rocprofv3 --pmc FETCH_SIZE -d DIR_F -o run --output-format csv -- python3 bench.py --pmc-probe",
             "    rocprofv3 --pmc WRITE_SIZE -d DIR_W -o run --output-format csv -- python3 bench.py --pmc-probe",
             "    python3 bench.py --pmc-summary DIR_F DIR_W", "",
             "The probe runs one decode step (nosa_decode_step) and one stand-alone attention "
             "(nosa_sparse_attend) on each of the eight layer caches at the first decode position.",
             "",
             f"Calibration: a plain copy reading and writing {CALIB_BYTES >> 20} MiB; "
             f"bytes per counter KiB: fetch {f_fetch * 1024:.1f}, write {f_write * 1024:.1f} "
             f"(factors {f_fetch:.3f} / {f_write:.3f} of the nominal 1024).", "",
             "| kernel | dispatches | FETCH_SIZE KiB | WRITE_SIZE KiB | fetched MB | written MB |",
             "|---|---:|---:|---:|---:|---:|"]
    traffic = {}
    for role in sorted(per):
        v = per[role]
        if "FETCH_SIZE" not in v or "WRITE_SIZE" not in v:
            continue
        fk, wk = float(np.mean(v["FETCH_SIZE"])), float(np.mean(v["WRITE_SIZE"]))
        fb, wb = fk * 1024 * f_fetch, wk * 1024 * f_write
        traffic[role] = fb + wb
        lines.append(f"| `{role}` | {len(v['FETCH_SIZE'])} | {fk:.0f} | {wk:.0f} | "
                     f"{fb / 1e6:.2f} | {wb / 1e6:.2f} |")

    def pick(part):
        ks = [k for k in traffic if part in k]
        if not ks:
            raise SystemExit(f"{part} not found")
        return traffic[ks[0]]
    step_t = pick("score_kernel") + pick("top_kernel") + pick("merge_kernel (decode step)")
    attn_t = pick("attend_kernel") + pick("merge_kernel (attention)")
    # the pooled-key build of each layer cache at setup reads every K token
    # once: B * L * Hkv * d bf16
    kcb = [k for k in per if "kc_build_kernel" in k]
    kc_lines = []
    if kcb:
        unique_k = w.batch * w.lens[0] * w.num_kv_heads * w.head_dim * 2
        fb = float(np.mean(per[kcb[0]]["FETCH_SIZE"])) * 1024 * f_fetch
        kc_lines = [f"- kc_build_fetch_bytes: {int(fb)} (one layer's full build)",
                    f"- kc_build_unique_k_bytes: {unique_k}",
                    f"- kc_build_fetch_over_unique_k: {fb / unique_k:.3f}"]
    lines += ["", "A decode step is its scoring, top and merge dispatches; the stand-alone "
              "attention its attention and merge dispatches (each merge dispatch is attributed "
              "to the launch before it).", "",
              f"- step_traffic_bytes: {int(step_t)}",
              f"- step_algorithmic_bytes: {int(step_alg)}",
              f"- step_traffic_over_algorithmic: {step_t / step_alg:.3f}",
              f"- attention_traffic_bytes: {int(attn_t)}",
              f"- attention_algorithmic_bytes: {int(attn_alg)}",
              f"- attention_traffic_over_algorithmic: {attn_t / attn_alg:.3f}",
              *kc_lines,
              f"- sources_sha256: {sources_sha256()}"]
    print("\n".join(lines))


def counter_table(dirs):
    """Markdown table of rocprofv3 counter runs: per library kernel, the mean
    per dispatch of every counter found in the given directories, then the
    figures derived from them where the counters are there (per SIMD of the
    1024; VALU busy counts one issue cycle per 4 clocks, as the quad-cycle
    counters do)."""
    import collections
    import numpy as np
    acc = collections.defaultdict(lambda: collections.defaultdict(list))
    order = []
    for d in dirs:
        for r in _csv_rows(d, "*counter_collection.csv"):
            name = r["Kernel_Name"].split("(")[0].replace("void ", "")
            if "nosa::" not in name:
                continue
            if name not in order:
                order.append(name)
            acc[name][r["Counter_Name"]].append(float(r["Counter_Value"]))
    counters = sorted({c for k in acc for c in acc[k]})
    print("| kernel | " + " | ".join(counters) + " |")
    print("|---|" + "---:|" * len(counters))
    for k in order:
        cells = [f"{np.mean(acc[k][c]):.4g}" if c in acc[k] else "" for c in counters]
        print(f"| `{k}` | " + " | ".join(cells) + " |")
    print("")
    for k in order:
        m = {c: float(np.mean(v)) for c, v in acc[k].items()}
        parts = []
        if "SQ_INSTS_VALU_MFMA_MOPS_BF16" in m:
            parts.append(f"bf16 MFMA work {m['SQ_INSTS_VALU_MFMA_MOPS_BF16'] * 512 / 1e9:.2f} GFLOP")
        if "SQ_VALU_MFMA_BUSY_CYCLES" in m:
            parts.append(f"MFMA busy {m['SQ_VALU_MFMA_BUSY_CYCLES'] / 1024 / 1e3:.1f}K cycles per SIMD")
        if "SQ_ACTIVE_INST_VALU" in m:
            parts.append(f"VALU issue {m['SQ_ACTIVE_INST_VALU'] * 4 / 1024 / 1e3:.1f}K cycles per SIMD")
        if "SQ_INSTS_VALU_TRANS_F32" in m and "SQ_INSTS_VALU" in m:
            parts.append(f"transcendental share of VALU instructions "
                         f"{m['SQ_INSTS_VALU_TRANS_F32'] / m['SQ_INSTS_VALU']:.2f}")
        if "GRBM_GUI_ACTIVE" in m:
            parts.append(f"GPU busy {m['GRBM_GUI_ACTIVE'] / 8 / 1e3:.1f}K cycles per XCD")
        if parts:
            print(f"- `{k}`: " + "; ".join(parts))
    print("")
    print(f"- sources_sha256: {sources_sha256()}")


def trace_summary(d):
    """Markdown rows (library kernels) of a rocprofv3 kernel_stats.csv, and
    the launch-level timeline of the decode step from the kernel trace:
    per-kernel duration and the gap before it, medians over the steps (the
    tracer itself stretches the gaps)."""
    import numpy as np
    print("| kernel | calls | average (us) | min (us) | max (us) | share of GPU time |")
    print("|---|---:|---:|---:|---:|---:|")
    for r in _csv_rows(d, "*kernel_stats.csv"):
        if "nosa::" not in r["Name"]:
            continue
        name = r["Name"].split("(")[0] if r["Name"].startswith("nosa::") else r["Name"].split("(nosa")[0]
        print(f"| `{name}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.2f} | "
              f"{float(r['MinNs']) / 1e3:.2f} | {float(r['MaxNs']) / 1e3:.2f} | "
              f"{float(r['Percentage']):.1f}% |")
    try:
        tr = _csv_rows(d, "*kernel_trace.csv")
    except SystemExit:
        tr = []
    ev = sorted((int(r["Start_Timestamp"]), int(r["End_Timestamp"]), r["Kernel_Name"]) for r in tr)
    seq = []  # (score, top, merge) triples that follow each other
    for i in range(len(ev) - 2):
        a, b, c = ev[i], ev[i + 1], ev[i + 2]
        if "score_kernel" in a[2] and "top_kernel" in b[2] and "merge_kernel" in c[2]:
            seq.append((a, b, c))
    if seq:
        dur = lambda k: np.median([(t[k][1] - t[k][0]) / 1e3 for t in seq])
        gap = lambda k: np.median([(t[k][0] - t[k - 1][1]) / 1e3 for t in seq])
        whole = np.median([(t[2][1] - t[0][0]) / 1e3 for t in seq])
        print("")
        print(f"Decode-step timeline under the tracer (medians over {len(seq)} steps, us): "
              f"score_kernel {dur(0):.2f} | gap {gap(1):.2f} | top_kernel {dur(1):.2f} | "
              f"gap {gap(2):.2f} | merge_kernel {dur(2):.2f} | whole step {whole:.2f}")
    print("")
    print(f"- sources_sha256: {sources_sha256()}")


def _cpu_model():
    try:
        with open("/proc/cpuinfo") as fh:
            for line in fh:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def cpu_baseline(w, budget_s):
    """The CPU reference as it stands, on host copies of layer 0 of the timed
    workload: consecutive decode steps from the first position, each the
    method's step as the GPU runs it -- append the pooled key the current
    token completes (the earlier keys are kept from the step before), score,
    pool, select, attend -- with every host thread (OpenMP over sequences and
    heads) for about budget_s seconds, then with one thread for a third of
    that.  Packing each step's live tokens for the reference is not timed."""
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import synth
    from oracle import oracle as ora

    wl = synth.Workload(**{**w.__dict__, "meta": {}})  # layer 0's seed
    inp = synth.make_inputs(wl, device="cuda")
    host = dict(k=inp["k"].cpu(), v=inp["v"].cpu(), cu_k_store=inp["cu_k_store"].cpu())
    q = synth.bits(inp["q"])
    del inp
    op = ora.Params(w.num_q_heads, w.num_kv_heads, w.head_dim, w.block_size, w.kernel, w.stride,
                    w.topk, w.window, locality=w.locality)
    nsteps = w.extra_tokens + 1
    k0, _, cu0 = synth.packed_live(host, w, -1)  # the tokens before the first position
    max_nc = ora.num_keys(max(w.lens) + w.extra_tokens, op)
    all_threads = ora.num_threads()

    def run(threads, budget):
        ora.set_num_threads(threads)
        kc = ora.compress_keys(op, synth.bits(k0), cu0.numpy(), max_nc=max_nc)
        n, spent = 0, 0.0
        while n < nsteps and spent < budget:
            k, v, cu = synth.packed_live(host, w, n)
            kb, vb, cun = synth.bits(k), synth.bits(v), cu.numpy()
            valid = np.array([L - 1 for L in (cun[1:] - cun[:-1])], np.int32)
            t0 = time.time()
            ora.append_keys(op, kb, cun, valid, kc)
            sc = ora.block_scores(op, q, None, kc, cun)
            sel, cnt = ora.select_blocks(op, sc, None, cun)
            ora.sparse_attend(op, q, None, kb, vb, cun, sel, cnt)
            spent += time.time() - t0
            n += 1
        return n, spent

    n, dt = run(all_threads, budget_s)
    n1, dt1 = run(1, budget_s / 3)
    ora.set_num_threads(all_threads)
    return {"value": round(w.batch * n / dt, 2), "unit": "tokens/s", "cores": all_threads,
            "kind": "oracle",
            "sample": f"{n} consecutive decode steps of {w.name} (batch {w.batch}, layer 0, "
                      f"positions 0..{n - 1}: pooled-key append, scoring, pooling, selection, "
                      f"attention) on the host, fp64 reference, OpenMP over (sequence, head)",
            "one_thread": {"value": round(w.batch * n1 / dt1, 2), "unit": "tokens/s",
                           "steps": n1},
            "cpu_model": _cpu_model(), "nproc": os.cpu_count()}


def ceiling_main(args):
    """Read ceilings of the device: 2 GiB read as a stream (pages in order)
    and as a gather of 32 KB pages in random order (the probe kernel of
    libnosa_ceiling.so, a sweep of workgroup counts, median of 5 launches
    each), and a 2 GiB device-to-device copy."""
    import ctypes
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import build
    if not os.path.exists(build.PROBE_LIB):
        raise SystemExit(f"{build.PROBE_LIB} is missing: build it first")
    lib = ctypes.CDLL(build.PROBE_LIB)
    lib.nosa_probe_read_pages.argtypes = [ctypes.c_void_p, ctypes.c_void_p, ctypes.c_int,
                                          ctypes.c_int, ctypes.c_void_p, ctypes.c_void_p]
    lib.nosa_probe_read_pages.restype = ctypes.c_int
    page, nbytes = 32768, 2 << 30
    npages = nbytes // page
    src = torch.empty(nbytes // 2, dtype=torch.int16, device="cuda").random_()
    gen = torch.Generator(device="cuda").manual_seed(7)
    orders = {"stream": torch.arange(npages, dtype=torch.int32, device="cuda"),
              "random_pages": torch.randperm(npages, generator=gen, device="cuda").to(torch.int32)}
    stream = torch.cuda.current_stream()
    res = {}
    for kind, order in orders.items():
        sweep = {}
        for wgs in (256, 512, 1024, 2048, 4096):
            sink = torch.empty(wgs * 4 * 64, dtype=torch.int32, device="cuda")
            launch = lambda: lib.nosa_probe_read_pages(src.data_ptr(), order.data_ptr(), npages,
                                                        wgs, sink.data_ptr(), stream.cuda_stream)
            assert launch() == 0
            torch.cuda.synchronize()
            ts = []
            for _ in range(5):
                e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
                e0.record(stream)
                launch()
                e1.record(stream)
                torch.cuda.synchronize()
                ts.append(e0.elapsed_time(e1))
            sweep[wgs] = round(nbytes / (float(np.median(ts)) * 1e-3) / 1e9, 1)
        best = max(sweep, key=sweep.get)
        res[kind] = {"gbs": sweep[best], "workgroups": best, "sweep_gbs": sweep,
                     "frac": round(sweep[best] / HBM_PEAK_GBS, 4)}
        print(f"[ceiling] {kind}: {sweep}", file=sys.stderr, flush=True)
    del src
    torch.cuda.empty_cache()
    copy = copy_bandwidth()
    out = {"metric": "device read ceilings (2 GiB)", "value": res["random_pages"]["gbs"],
           "unit": "GB/s", "n_gpus": 1, "higher_is_better": True, "dtype": "bytes",
           "data": "random 16-bit words", "config": {"workload": "read-ceilings-2g",
                                                      "page_bytes": page, "bytes": nbytes},
           "stream_read": res["stream"], "random_page_gather": res["random_pages"],
           "copy_2g": {"gbs": round(copy, 1), "frac": round(copy / HBM_PEAK_GBS, 4),
                       "note": "bytes read + bytes written"},
           "peak_gbs": HBM_PEAK_GBS,
           "device": torch.cuda.get_device_name(0)}
    print(json.dumps(out), flush=True)


def timeline_main(w, args):
    """Where a decode step's time goes: the decode kernels built with
    wall-clock stamps (libnosa_timeline.so) run graph-captured steps of
    workload w over 16 layer caches; the stamps of a replay's last step
    (thread 0 of each workgroup at fixed points of its launch) give, relative
    to the first scoring workgroup's start, each phase's median over the
    workgroups and the launch ends.  Medians over 20 decode positions."""
    import ctypes
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import build, nosa, synth
    if not os.path.exists(build.TIMELINE_LIB):
        raise SystemExit(f"{build.TIMELINE_LIB} is missing: build it first")
    nosa.LIB_PATH = build.TIMELINE_LIB
    L = nosa.lib()
    L.nosa_timeline_read.argtypes = [ctypes.c_int, ctypes.c_void_p]
    for f in ("nosa_timeline_read", "nosa_timeline_clear", "nosa_timeline_clock_khz"):
        getattr(L, f).restype = ctypes.c_int
    khz = L.nosa_timeline_clock_khz()
    assert khz > 0
    nl = 16
    nsteps = w.extra_tokens + 1
    layers = build_layers(w, nsteps, nlayers=nl, full_kc=True)
    B, Hq, d = w.batch, w.num_q_heads, w.head_dim
    cu_at = [synth.cu_from_lens([x + t for x in w.lens], "cuda") for t in range(nsteps)]
    maxL = max(w.lens) + nsteps - 1
    ws = torch.zeros(nosa.nosa_workspace_size(layers[0]["p"], B, 1, maxL), dtype=torch.uint8,
                     device="cuda")
    out = torch.empty(B, Hq, d, device="cuda")
    lse = torch.empty(B, Hq, device="cuda")

    def step(i, t):
        ly = layers[i % nl]
        nosa.nosa_decode_step(ly["p"], ly["kv"], ly["inp"]["q"], cu_at[t], B, maxL, out, lse, ws)

    for i in range(32):
        step(i, i % nsteps)
    torch.cuda.synchronize()
    stamps = np.zeros((3, 8192, 16), dtype=np.uint64)
    stream = torch.cuda.current_stream()
    per_rep, step_us = [], []
    for rep in range(20):
        t = (rep * 13) % nsteps
        g = torch.cuda.CUDAGraph()
        with torch.cuda.graph(g):
            for i in range(nl):
                step(i, t)
        g.replay()
        torch.cuda.synchronize()
        assert L.nosa_timeline_clear() == 0
        e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        e0.record(stream)
        g.replay()
        e1.record(stream)
        torch.cuda.synchronize()
        step_us.append(e0.elapsed_time(e1) * 1e3 / nl)
        for k in range(3):
            assert L.nosa_timeline_read(k, stamps[k].ctypes.data) == 0
        us = stamps.astype(np.float64) * 1e3 / khz  # ticks -> us
        sc, tp, mg = us[0], us[1], us[2]
        sc_done = sc[sc[:, 2] > 0]
        score_rows = sc_done[sc_done[:, 7] == 0]
        top_done = tp[tp[:, 5] > 0]
        top_rows = top_done[top_done[:, 7] == 0]
        win_rows = top_done[top_done[:, 7] > 0]
        mg_done = mg[mg[:, 1] > 0]
        t0 = sc_done[:, 0].min()
        r = {"scoring_start_median": np.median(score_rows[:, 0]) - t0,
             "scoring_keys_multiplied": np.median(score_rows[:, 1]) - t0,
             "scoring_end": sc_done[:, 2].max() - t0,
             "attention_start": top_done[:, 0].min() - t0,
             "top_start_median": np.median(top_rows[:, 0]) - t0,
             "top_bounds_in": np.median(top_rows[:, 12]) - t0,
             "top_wave0_log_sum_exp": np.median(top_rows[:, 6]) - t0,
             "top_log_sum_exp": np.median(top_rows[:, 1]) - t0,
             "top_importance": np.median(top_rows[:, 2]) - t0,
             "select_range": np.median(top_rows[:, 8]) - t0,
             "select_first_digit": np.median(top_rows[:, 9]) - t0,
             "select_last_digit": np.median(top_rows[:, 10]) - t0,
             "select_counts_shared": np.median(top_rows[:, 11]) - t0,
             # point 15: stamped when the selector runs a digit level after the first
             "select_more_levels_share": float(np.mean(top_rows[:, 15] > 0)),
             "top_selection": np.median(top_rows[:, 3]) - t0,
             "top_pages_attended": np.median(top_rows[:, 4]) - t0,
             "top_partial_stored": np.median(top_rows[:, 5]) - t0,
             "top_end": top_rows[:, 5].max() - t0,
             "window_end": win_rows[:, 5].max() - t0 if len(win_rows) else float("nan"),
             "attention_end": top_done[:, 5].max() - t0,
             "merge_start": mg_done[:, 0].min() - t0,
             "merge_end": mg_done[:, 1].max() - t0}
        # placement: the XCD of each workgroup against blockIdx % 8, and the
        # top workgroups' ends per XCD and per count of them sharing a CU
        idx = np.nonzero((stamps[1][:, 5] > 0) & (stamps[1][:, 7] == 0))[0]
        xcc = stamps[1][idx, 13].astype(np.int64) & 15
        hw = stamps[1][idx, 14].astype(np.int64)
        cu_key = xcc * 256 + ((hw >> 8) & 0xff)  # XCD, engine, array, compute unit
        _, inv, cnt = np.unique(cu_key, return_inverse=True, return_counts=True)
        ends = tp[idx, 5] - t0
        r["top_on_blockidx_xcd"] = float(np.mean(xcc == (idx % 8)))
        # XCD of blockIdx 0 .. 7 in each launch (the same blockIdx % 8 runs on
        # one XCD within a launch; the first one's XCD may differ per launch)
        for k, name in ((0, "scoring"), (1, "attention"), (2, "merge")):
            done = stamps[k][:, 2 if k == 0 else (5 if k == 1 else 1)] > 0
            ids = [int(stamps[k][b, 13]) & 15 if done[b] else -1 for b in range(8)]
            r[f"xcd_of_blockidx0_{name}"] = ids[0]
            r[f"xcd_rotation_consistent_{name}"] = float(all(
                i < 0 or i == (ids[0] + b) % 8 for b, i in enumerate(ids)))
        offs = [r[f"xcd_of_blockidx0_{n}"] for n in ("scoring", "attention", "merge")]
        r["xcd_offsets_equal_share"] = float(len(set(offs)) == 1)
        print(json.dumps({"rep": rep, "xcd_of_blockidx0": offs}), file=sys.stderr, flush=True)
        if rep == 0:
            xmap = {int(b): sorted({int(v) for v in xcc[idx % 8 == b]}) for b in range(8)}
            raw = [(int(i), int(stamps[1][i, 13]), int(stamps[1][i, 14])) for i in idx[:16]]
            print(json.dumps({"blockidx_mod8_to_xcc": xmap, "raw_id_hw": raw}), file=sys.stderr,
                  flush=True)
        for x in range(8):
            sel = xcc == x
            r[f"top_end_xcd{x}"] = float(ends[sel].max()) if sel.any() else float("nan")
        for n in (1, 2, 3):
            sel = cnt[inv] == n
            r[f"top_end_median_cu_with_{n}"] = float(np.median(ends[sel])) if sel.any() else float("nan")
            r[f"top_share_cu_with_{n}"] = float(np.mean(sel))
        r["gap_scoring_to_attention"] = r["attention_start"] - r["scoring_end"]
        r["gap_attention_to_merge"] = r["merge_start"] - r["attention_end"]
        per_rep.append(r)
    med = {k: round(float(np.median([r[k] for r in per_rep])), 2) for k in per_rep[0]}
    for k in list(med):
        if "share" in k or k.startswith("top_on_") or k.startswith("xcd_rotation"):
            med[k] = round(float(np.mean([r[k] for r in per_rep])), 3)
    res = {"metric": "decode step timeline", "value": med["merge_end"], "unit": "us from the first scoring workgroup's start",
           "n_gpus": 1, "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.name, "batch": w.batch, "context": max(w.lens), "positions": 20,
                      "layer_caches": nl},
           "phases_us": med, "instrumented_us_per_step": round(float(np.median(step_us)), 2),
           "wall_clock_khz": khz}
    print(json.dumps(res), flush=True)


def timeline_prefill_main(w, args):
    """Where a prefill chunk's time goes: the chain nosa_block_scores ->
    nosa_select_blocks -> nosa_sparse_attend with the prefill kernels built
    with wall-clock stamps (libnosa_timeline.so): per launch, when its
    workgroups start and leave (first, median, last) and the share of the
    launch each workgroup is resident on average.  Medians over 5 runs of the
    chain."""
    import ctypes
    import math
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import build, nosa, synth
    if not os.path.exists(build.TIMELINE_LIB):
        raise SystemExit(f"{build.TIMELINE_LIB} is missing: build it first")
    nosa.LIB_PATH = build.TIMELINE_LIB
    L = nosa.lib()
    L.nosa_timeline_read_prefill.argtypes = [ctypes.c_int, ctypes.c_void_p]
    for f in ("nosa_timeline_read_prefill", "nosa_timeline_clear_prefill", "nosa_timeline_clock_khz"):
        getattr(L, f).restype = ctypes.c_int
    khz = L.nosa_timeline_clock_khz()
    assert khz > 0
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
    mq, max_nb = math.ceil(maxLq / 64), math.ceil(maxL / 64)
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

    for _ in range(3):
        chain()
    torch.cuda.synchronize()
    names = {0: "scoring_pass1", 1: "scoring_pass2", 3: "pooling", 2: "attention"}
    stamps = np.zeros((8192, 4), dtype=np.uint64)
    runs = []
    for rep in range(5):
        assert L.nosa_timeline_clear_prefill() == 0
        chain()
        torch.cuda.synchronize()
        t0, r = None, {}
        for k in (0, 1, 3, 2):
            assert L.nosa_timeline_read_prefill(k, stamps.ctypes.data) == 0
            done = stamps[(stamps[:, 0] > 0) & (stamps[:, 1] > 0)].astype(np.float64) * 1e3 / khz
            if len(done) == 0:
                continue
            if t0 is None:
                t0 = done[:, 0].min()
            st, en = done[:, 0] - t0, done[:, 1] - t0
            xcc = stamps[(stamps[:, 0] > 0) & (stamps[:, 1] > 0)][:, 2].astype(np.int64) & 15
            span = en.max() - st.min()
            r[names[k]] = {"workgroups": int(len(done)), "first_start": st.min(),
                           "median_start": float(np.median(st)), "last_start": st.max(),
                           "median_end": float(np.median(en)), "last_end": en.max(),
                           "resident_share": float(np.mean(en - st) / span) if span > 0 else 1.0}
            for x in range(8):
                sel_x = xcc == x
                r[names[k]][f"median_end_xcd{x}"] = float(np.median(en[sel_x])) if sel_x.any() else float("nan")
                r[names[k]][f"last_end_xcd{x}"] = float(en[sel_x].max()) if sel_x.any() else float("nan")
        runs.append(r)
    med = {n: {k: round(float(np.median([r[n][k] for r in runs])), 3) for k in runs[0][n]}
           for n in runs[0]}
    res = {"metric": "prefill chunk timeline", "value": med[list(med)[-1]]["last_end"],
           "unit": "us from the first scoring workgroup's start", "n_gpus": 1,
           "higher_is_better": False, "dtype": "bf16", "data": "synthetic",
           "config": {"workload": w.name, "queries": maxLq, "context": maxL, "runs": 5},
           "launches_us": med, "wall_clock_khz": khz}
    print(json.dumps(res), flush=True)


def chip_probes_main(args):
    """Costs of this chip that the design rests on (the machine probes of
    libnosa_ceiling.so; medians of repeated launches): how far VALU work and
    MFMAs overlap in the prefill scoring step's instruction mix, the LDS read
    bandwidth, a hand-off of partials inside one launch against a second
    launch, and the latency of a dependent device-memory load."""
    import ctypes
    import numpy as np
    import torch
    from block_sparse_attention_nosa_amd import build
    if not os.path.exists(build.PROBE_LIB):
        raise SystemExit(f"{build.PROBE_LIB} is missing: build it first")
    lib = ctypes.CDLL(build.PROBE_LIB)
    vp, i32 = ctypes.c_void_p, ctypes.c_int
    lib.nosa_probe_mix.argtypes = [i32, i32, i32, vp, vp]
    lib.nosa_probe_lds_read.argtypes = [i32, i32, vp, vp]
    lib.nosa_probe_handoff.argtypes = [i32, i32, vp, vp, vp, vp]
    lib.nosa_probe_chase.argtypes = [vp, i32, i32, i32, i32, i32, vp, vp, vp]
    lib.nosa_probe_wall_clock_khz.argtypes = []
    for f in ("nosa_probe_mix", "nosa_probe_lds_read", "nosa_probe_handoff", "nosa_probe_chase",
              "nosa_probe_wall_clock_khz"):
        getattr(lib, f).restype = ctypes.c_int
    stream = torch.cuda.current_stream()
    sh = stream.cuda_stream

    def timed(launch, reps=5):
        assert launch() == 0
        torch.cuda.synchronize()
        ts = []
        for _ in range(reps):
            e0, e1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            e0.record(stream)
            assert launch() == 0
            e1.record(stream)
            torch.cuda.synchronize()
            ts.append(e0.elapsed_time(e1) * 1e3)  # us
        return float(np.median(ts))

    # instruction mix: 512 workgroups (two per CU, two waves per SIMD); per
    # wave and iteration 64 MFMAs (1024 MFMA cycles) and the VALU work of
    # 64 products; per SIMD an iteration runs two waves' worth
    wgs, iters = 512, 2000
    sink = torch.empty(wgs * 256, dtype=torch.float32, device="cuda")
    names = {0: "mfma_and_dependent_valu", 1: "mfma_only", 2: "valu_only", 3: "mfma_and_independent_valu"}
    mix = {}
    for m, name in names.items():
        us = timed(lambda: lib.nosa_probe_mix(m, wgs, iters, sink.data_ptr(), sh))
        mix[name] = round(us * 1e3 / iters, 1)  # ns per iteration per SIMD
    t1, t2, t3 = mix["mfma_only"], mix["valu_only"], mix["mfma_and_independent_valu"]
    mix["unit"] = "ns per iteration per SIMD (two waves, 128 MFMAs)"
    mix["independent_overlap_of_mfma_time"] = round((t1 + t2 - t3) / t1, 3)
    # LDS reads: 512 workgroups, 32 KB per wave per iteration
    lsink = torch.empty(wgs * 256, dtype=torch.int32, device="cuda")
    liters = 4000
    us = timed(lambda: lib.nosa_probe_lds_read(wgs, liters, lsink.data_ptr(), sh))
    lds_bytes = wgs * 4 * liters * 32 * 1024
    lds = {"bytes_per_ns_per_cu": round(lds_bytes / (us * 1e3) / torch.cuda.get_device_properties(0).multi_processor_count, 1),
           "total_tb_s": round(lds_bytes / (us * 1e-6) / 1e12, 1)}
    # hand-off of 16 groups of 16 workgroups' 4 KB partials
    groups = 16
    part = torch.zeros(groups * 16 * 1024, dtype=torch.float32, device="cuda")
    counter = torch.zeros(groups, dtype=torch.int32, device="cuda")
    out = torch.zeros(groups * 1024, dtype=torch.float32, device="cuda")
    want = torch.tensor([16 * 16 * g + 136 for g in range(groups)], dtype=torch.float32)
    hand = {}
    for mode, name in ((0, "release_acquire_fences"), (1, "coherent_stores_no_fence"), (2, "two_launches")):
        out.zero_()
        us = timed(lambda: lib.nosa_probe_handoff(mode, groups, part.data_ptr(), counter.data_ptr(),
                                                  out.data_ptr(), sh), reps=11)
        ok = bool(torch.equal(out.view(groups, 1024).cpu(), want[:, None].expand(groups, 1024)))
        hand[name] = {"us": round(us, 2), "sums_correct": ok}
    # dependent loads: a random cycle through an array, walked by one wave
    # and timed inside the launch.  Lines in the XCD's L2: a 1 MB array, the
    # timed hops walked once before (all its lines fit); in the Infinity
    # Cache: 64 MB, 100000 hops walked once before (12.8 MB of lines, beyond
    # the 4 MB L2, within the 256 MB Infinity Cache); in HBM only: 1 GiB, a
    # part of the cycle that no walk has touched.  The chain's end is
    # checked against the cycle: next[perm[j]] = perm[j + 1].
    khz = lib.nosa_probe_wall_clock_khz()
    assert khz > 0
    zero = torch.zeros(64, dtype=torch.int32, device="cuda")
    cout = torch.zeros(2, dtype=torch.int64, device="cuda")
    chase = {"wall_clock_khz": khz}
    ends_ok = True
    for level, n, steps, warm in (("l2", 1 << 18, 20000, True), ("infinity_cache", 1 << 24, 100000, True),
                                  ("hbm", 1 << 28, 20000, False)):
        gen = torch.Generator(device="cuda").manual_seed(11)
        perm = torch.randperm(n, generator=gen, device="cuda").to(torch.int32)
        nxt = torch.empty(n, dtype=torch.int32, device="cuda")
        nxt[perm.long()] = torch.roll(perm, -1)
        permh = perm.cpu()
        if not warm:  # evict the writes and reads above from the Infinity Cache
            flush = torch.ones(1 << 27, dtype=torch.int32, device="cuda")
            assert int(flush.sum()) == 1 << 27
            del flush
        res_l = {"array_mb": n * 4 / 2**20, "hops": steps}
        for vec, name in ((1, "vector_load_ns"), (0, "scalar_load_ns")):
            ns = []
            for rep in range(3):
                j = rep * 2 * steps + (0 if vec else 6 * steps)  # a fresh part of the cycle (hbm)
                start = int(permh[j])
                assert lib.nosa_probe_chase(nxt.data_ptr(), start, steps if warm else 0, start, steps, vec,
                                            zero.data_ptr(), cout.data_ptr(), sh) == 0
                torch.cuda.synchronize()
                end, ticks = (int(v) for v in cout.cpu())
                ends_ok &= end == int(permh[(j + steps) % n])
                ns.append(ticks * 1e6 / khz / steps)
            res_l[name] = round(float(np.median(ns)), 1)
        chase[level] = res_l
        del perm, nxt, permh
    chase["ends_match_cycle"] = ends_ok
    res = {"metric": "chip probes", "value": mix["mfma_and_dependent_valu"], "unit": mix["unit"],
           "n_gpus": 1, "higher_is_better": False, "dtype": "bf16/fp32", "data": "synthetic",
           "config": {"workload": "chip-probes", "workgroups": wgs},
           "instruction_mix": mix, "lds_read": lds, "handoff_16x16_workgroups": hand,
           "dependent_load": chase, "device": torch.cuda.get_device_name(0)}
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
