"""Build libbitnet_mi355x.so (gfx950) in-tree with hipcc.

    python -m ternary_weight_linear_bit_amd.build

Each .hip source is compiled to an object in parallel, then linked into one
shared library next to this file.  hipcc cross-compiles for gfx950 without a GPU.
"""

from __future__ import annotations

import os
import shutil
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
BUILD = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libbitnet_mi355x.so")
SOURCES = ("api.hip", "wq.hip", "aq.hip", "gemv.hip", "gemm.hip", "lut.hip", "chain.hip")
# bench-only diagnostics (int8 matrix-core rate, HBM read rates, launch cost), their
# own library: not part of the ABI
PROBE_SRCS = [os.path.join(PKG, "bench_probe", f) for f in ("mfma_probe.hip", "hbm_probe.hip")]
PROBE_LIB = os.path.join(PKG, "libbitnet_bench_probe.so")

HIPCC = os.environ.get("HIPCC", shutil.which("hipcc") or "/opt/rocm/bin/hipcc")
FLAGS = [
    "--offload-arch=gfx950",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-ffp-contract=off",              # the rescale and quantisers must round exactly as written
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    "-Wall",
    "-I", os.path.join(ROOT, "include"),
    "-I", CSRC,
]


# Per-source flags: the decode kernel's leading scalar arguments are preloaded
# into SGPRs at wave launch (gfx950 kernarg preload; the compiler adds the
# fallback preamble for firmware without it).
EXTRA = {"gemv.hip": ("-mllvm", "-amdgpu-kernarg-preload-count=10")}


def _run(cmd):
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError("build failed: " + " ".join(cmd) + "\n" + r.stdout + r.stderr)
    return r


def build(verbose: bool = False) -> str:
    os.makedirs(BUILD, exist_ok=True)
    objs = [os.path.join(BUILD, s.replace(".hip", ".o")) for s in SOURCES]
    cmds = [[HIPCC, *FLAGS, *EXTRA.get(s, ()), "-c", os.path.join(CSRC, s), "-o", o]
            for s, o in zip(SOURCES, objs)]
    with ThreadPoolExecutor(max_workers=min(len(cmds), os.cpu_count() or 4)) as ex:
        for r in ex.map(_run, cmds):
            if verbose and (r.stdout or r.stderr):
                print(r.stdout + r.stderr)
    tmp = LIB + ".tmp"
    _run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", *objs, "-o", tmp])
    os.replace(tmp, LIB)
    tmp = PROBE_LIB + ".tmp"
    # the matrix-core probe keeps its accumulators in arch VGPRs: with them in
    # AGPRs, two waves per SIMD measured 1207 instead of 2046 int8 ops per clock
    _run([HIPCC, *FLAGS, "-mllvm", "-amdgpu-mfma-vgpr-form=1", "-shared", *PROBE_SRCS, "-o", tmp])
    os.replace(tmp, PROBE_LIB)
    return LIB


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
