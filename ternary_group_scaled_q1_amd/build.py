"""Build liblowbit.so (HIP kernels for gfx950 + host packer + C ABI) in-tree,
and libprobes.so, the benchmark's platform probes (plain streaming-read,
MFMA and empty kernels; no part of the product path).

    python -m ternary_group_scaled_q1_amd.build      # or build() from Python
"""
from __future__ import annotations

import os
import shutil
import subprocess
import sys
import tempfile

PKG = os.path.dirname(os.path.abspath(__file__))
CSRC = os.path.join(PKG, "csrc")
LIB = os.path.join(PKG, "liblowbit.so")
PROBES_LIB = os.path.join(PKG, "libprobes.so")
PROBES_SOURCES = ["probes.hip"]
ARCH = "gfx950"

SOURCES = ["api.hip", "noalloc.hip", "gemv.hip", "gemv_wide.hip", "gemv_split.hip", "gemv_kslice.hip", "gemv_tq5.hip", "gemm.hip", "device_props.cpp", "pack.cpp"]

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}", "-O3", "-std=c++17", "-fPIC", "-Wall", "-Wno-unused-function",
    # No packed-FP32 instructions in device code.
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # Every wave runs its prologue (the first loads of x and of the weight
    # ring) at raised issue priority and drops to normal priority (s_setprio)
    # where its main loop begins, so the first loads of all waves on a SIMD
    # leave before any wave's compute: 1-2% on the decode sweeps, neutral on
    # the GEMMs.
    "-mllvm", "-amdgpu-set-wave-priority",
]


def _hipcc() -> str:
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", shutil.which("hipcc")):
        if c and os.path.exists(c):
            return c
    raise RuntimeError("hipcc not found (ROCm is required to build the library)")


# Per-source extra flags: the GEMM keeps its MFMA accumulators in VGPRs (the
# per-group fp32 scale epilogue then needs no moves out of AGPRs); the
# K-sliced GEMV is scheduled for instruction-level parallelism rather than
# occupancy (its 16-token launches 4-8% faster; the same strategy made the
# one-token staged kernel 3-6% slower and left the split kernel and the
# GEMMs unchanged, so it stays on this file only).
EXTRA_FLAGS = {"gemm.hip": ["-mllvm", "-amdgpu-mfma-vgpr-form"],
               "gemv_kslice.hip": ["-mllvm", "-amdgpu-sched-strategy=max-ilp"]}


def build(verbose: bool = False, jobs: int = 4) -> str:
    _build_lib(SOURCES, LIB, verbose, jobs)
    _build_lib(PROBES_SOURCES, PROBES_LIB, verbose, jobs)
    return LIB


def _build_lib(sources, lib, verbose, jobs):
    hipcc = _hipcc()
    tmp = tempfile.mkdtemp(prefix="lowbit_build_")
    try:
        objs, procs = [], []
        for src in sources:
            obj = os.path.join(tmp, src + ".o")
            lang = ["-x", "hip"] if src.endswith(".cpp") else []
            cmd = [hipcc, *HIPCC_FLAGS, *EXTRA_FLAGS.get(src, []), *lang, "-c", os.path.join(CSRC, src), "-o", obj]
            if verbose:
                print(" ".join(cmd), flush=True)
            procs.append((src, subprocess.Popen(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT)))
            objs.append(obj)
            if len(procs) >= jobs:
                _wait(procs.pop(0))
        while procs:
            _wait(procs.pop(0))
        out_tmp = lib + ".tmp"
        cmd = [hipcc, f"--offload-arch={ARCH}", "-shared", "-fPIC", *objs, "-o", out_tmp, "-lpthread"]
        if verbose:
            print(" ".join(cmd), flush=True)
        r = subprocess.run(cmd, stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True)
        if r.returncode != 0:
            raise RuntimeError("link failed:\n" + r.stdout)
        os.replace(out_tmp, lib)
    finally:
        shutil.rmtree(tmp, ignore_errors=True)
    return lib


def _wait(item):
    src, p = item
    out, _ = p.communicate()
    text = out.decode(errors="replace")
    # hipcc's host pass does not know the device-only target feature; drop that note.
    text = "\n".join(l for l in text.splitlines() if "packed-fp32-ops" not in l)
    if p.returncode != 0:
        raise RuntimeError(f"compiling {src} failed:\n{text}")
    if text.strip():
        print(text, file=sys.stderr)


if __name__ == "__main__":
    print(build(verbose="-v" in sys.argv))
