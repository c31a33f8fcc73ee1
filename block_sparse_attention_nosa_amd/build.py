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


def _compile(cmd, tmp, lib, what, verbose):
    r = subprocess.run(cmd, cwd=ROOT, capture_output=True, text=True)
    if r.returncode != 0:
        sys.stderr.write(r.stdout + r.stderr)
        raise RuntimeError(f"hipcc failed building {what}")
    if verbose:
        sys.stderr.write(r.stderr)
    os.replace(tmp, lib)


def build(verbose: bool = False) -> str:
    _compile(hipcc_cmd(LIB + ".tmp"), LIB + ".tmp", LIB, "libnosa.so", verbose)
    probe = hipcc_cmd(PROBE_LIB + ".tmp")
    probe = [a for a in probe if a not in SOURCES]
    probe[probe.index("-o"):probe.index("-o")] = PROBE_SOURCES
    _compile(probe, PROBE_LIB + ".tmp", PROBE_LIB, "libnosa_ceiling.so", verbose)
    return LIB


if __name__ == "__main__":
    print(build(verbose=True))
