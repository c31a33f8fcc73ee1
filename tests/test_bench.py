"""The benchmark's host logic without a GPU: the one-GPU contract, the byte and
flop accounting behind its rates (against sums worked out by hand from the
workload definitions), and the rule that counter traffic is reported only for
the sources it was measured on."""
import os
import subprocess
import sys

import pytest

import bench
from block_sparse_attention_nosa_amd import synth

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_step_bytes_of_the_16k_workload():
    """First step of the batch-8 16K workload, per (sequence, KV head): 1023
    pooled keys (256 B each); 80 kept blocks of which the last holds 1 token:
    5057 tokens of K and V (512 B per token); q (8 heads x 256 B), out (8 x
    512 B) and lse (8 x 4 B); the append reads 32 tokens and writes a key."""
    w = synth.config(2)
    lens = [L for L in w.lens]
    per_pair_attn = 5057 * 512 + 8 * 256 + 8 * 512 + 8 * 4
    per_pair = 1023 * 256 + per_pair_attn
    step, attn = bench.algorithmic_bytes(w, lens, append=False)
    assert attn == 16 * per_pair_attn
    assert step == 16 * per_pair == 45_715_968
    step_a, _ = bench.algorithmic_bytes(w, lens, append=True)
    assert step_a - step == 16 * (32 * 256 + 256)


def test_prefill_flops_of_the_131072_chunk():
    """The 2048-query chunk at the end of 131072 tokens: each query scores the
    pooled keys it sees (about 8100) for 16 heads, and attends 80 blocks (the
    last one causal) -- about 68 and 86 GFLOP."""
    w = synth.config(5)
    fs, fa = bench.prefill_flops(w)
    p0 = 131072 - 2048
    nc = sum((p + 1 - 32) // 16 + 1 for p in range(p0, 131072))
    assert fs == 2.0 * 128 * nc * 16
    assert 67e9 < fs < 69e9 and 85e9 < fa < 87e9


def test_traffic_is_reported_only_for_its_sources(monkeypatch):
    assert bench.recorded_traffic("decode-varlen-b32", "step") is None  # not measured there
    monkeypatch.setattr(bench, "sources_sha256", lambda: "0" * 64)
    assert bench.recorded_traffic("decode-b8-16k", "step") is None  # kernels changed since
    assert bench.trace_average_us(bench.TRACE_FILE, "top_kernel<") is None


def test_timed_positions_cover_every_decode_position():
    """Whatever the number of timed steps, the replays' steps run through all
    256 decode positions in order, so appending steps (one pooled key every 16
    tokens) and steps that start a new block are timed too."""
    import math
    w = synth.config(2)
    for steps in (1, 20, 256, 2048):
        replays = max(5, math.ceil(256 / steps))
        pos = bench.step_positions(256, steps, replays)
        assert len(pos) == steps * replays
        assert set(pos) == set(range(256)), steps
        assert pos == sorted(pos)
        lens = [[L + t for L in w.lens] for t in pos]
        assert any((l[0] - w.kernel) % w.stride == 0 for l in lens)
        assert any((l[0] - 1) % w.block_size == 0 for l in lens)
