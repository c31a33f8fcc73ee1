"""The stamped build of the decode kernels (libnosa_timeline.so, the
benchmark's --timeline mode) on the smallest decode workload: every phase of
a step is stamped, in the order the step's dependencies impose (a launch
starts after the one before it has ended; inside the attention launch the
log-sum-exp, the importance, the selection, the pages and the partial follow
each other).  A process of its own: the mode loads the stamped library in
place of libnosa.so."""
import json
import math
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.gpu
def test_timeline_phases_in_dependency_order():
    from block_sparse_attention_nosa_amd import build
    if not os.path.exists(build.TIMELINE_LIB):
        pytest.fail(f"{build.TIMELINE_LIB} is missing: build it first")
    print("case: bench.py --timeline --config 1", flush=True)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--timeline", "--config", "1"],
                       cwd=ROOT, capture_output=True, text=True, timeout=240)
    assert r.returncode == 0, r.stderr[-3000:]
    line = [l for l in r.stdout.splitlines() if l.startswith("{")][-1]
    res = json.loads(line)
    ph = res["phases_us"]
    order = ["scoring_keys_multiplied", "scoring_end", "attention_start", "top_start_median",
             "top_log_sum_exp", "top_importance", "select_range", "select_first_digit",
             "select_counts_shared", "top_selection", "top_pages_attended", "top_partial_stored",
             "top_end", "merge_start", "merge_end"]
    vals = [ph[k] for k in order]
    assert all(math.isfinite(v) and v >= 0 for v in vals), ph
    for a, b, va, vb in zip(order, order[1:], vals, vals[1:]):
        assert va <= vb + 0.01, (a, va, b, vb)
    assert ph["gap_scoring_to_attention"] > 0 and ph["gap_attention_to_merge"] > 0, ph
    assert res["instrumented_us_per_step"] > 0
