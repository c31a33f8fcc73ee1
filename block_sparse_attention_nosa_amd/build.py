"""Builds the HIP library libnosa.so in-tree for gfx950 with hipcc.

    python -m block_sparse_attention_nosa_amd.build
"""
from __future__ import annotations

import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "libnosa.so")
SOURCES = [os.path.join(CSRC, "nosa_kernels.hip"), os.path.join(CSRC, "nosa_prefill.hip"),
           os.path.join(CSRC, "nosa_front.hip"), os.path.join(CSRC, "nosa_api.cpp")]
ARCH = "gfx950"


def hipcc_cmd(out=LIB):
    return ["hipcc", f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-shared",
            # no packed-fp32 instructions anywhere in the device code
            "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
            "-Wall", "-Wno-unused-function",
            "-I", os.path.join(ROOT, "include"), *SOURCES, "-o", out]


# The benchmark's machine probes (read ceilings, chip costs): a library of its own, not part of libnosa.so.
PROBE_SOURCES = [os.path.join(CSRC, "probe_ceiling.hip"), os.path.join(CSRC, "probe_chip.hip")]
PROBE_LIB = os.path.join(PKG, "libnosa_ceiling.so")


# The benchmark's timeline mode: the same sources with wall-clock stamps in the
# decode kernels (NOSA_TIMELINE), a library of its own.
TIMELINE_LIB = os.path.join(PKG, "libnosa_timeline.so")


def _compile(cmds, verbose):
    """Runs the (cmd, tmp, lib, what) compilations in parallel; each library
    is moved into place when its compilation succeeded."""
    procs = [(subprocess.Popen(cmd, cwd=ROOT, stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True),
              tmp, lib, what) for cmd, tmp, lib, what in cmds]
    failed = []
    for p, tmp, lib, what in procs:
        out, err = p.communicate()
        if p.returncode != 0:
            sys.stderr.write(out + err)
            failed.append(what)
            continue
        if verbose:
            sys.stderr.write(err)
        os.replace(tmp, lib)
    if failed:
        raise RuntimeError("hipcc failed building " + ", ".join(failed))


def build(verbose: bool = False) -> str:
    probe = hipcc_cmd(PROBE_LIB + ".tmp")
    probe = [a for a in probe if a not in SOURCES]
    probe[probe.index("-o"):probe.index("-o")] = PROBE_SOURCES
    timeline = hipcc_cmd(TIMELINE_LIB + ".tmp")
    timeline.insert(timeline.index("-I"), "-DNOSA_TIMELINE")
    _compile([(hipcc_cmd(LIB + ".tmp"), LIB + ".tmp", LIB, "libnosa.so"),
              (probe, PROBE_LIB + ".tmp", PROBE_LIB, "libnosa_ceiling.so"),
              (timeline, TIMELINE_LIB + ".tmp", TIMELINE_LIB, "libnosa_timeline.so")], verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
