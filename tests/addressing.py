"""Drives the bounds-checked host replica of the kernels' address arithmetic
(tests/replica/kernel_addressing.cpp) with the plans the library's own
planner picks (lowbit_gemv_plan / lowbit_gemm_plan).  Needs no GPU: with no
device the planner assumes 256 compute units and one workgroup per CU where
it would ask the runtime for occupancy."""
from __future__ import annotations

import hashlib
import os
import subprocess
import tempfile

import ternary_group_scaled_q1_amd as lb

HERE = os.path.dirname(os.path.abspath(__file__))
SRC = os.path.join(HERE, "replica", "kernel_addressing.cpp")
FLAGS = ["-std=c++17", "-O1", "-g", "-fsanitize=address,undefined", "-fno-sanitize-recover=undefined",
         "-fno-omit-frame-pointer", "-Wall", "-Wextra"]
SLOTS = 256  # stream-K workgroup slots of the GEMM: one per compute unit of an MI355X


def build_replica() -> str:
    """Compile the replica with AddressSanitizer and UBSan (cached by source hash)."""
    digest = hashlib.sha256(open(SRC, "rb").read() + " ".join(FLAGS).encode()).hexdigest()[:16]
    out = os.path.join(tempfile.gettempdir(), f"lowbit_kernel_addressing_{digest}")
    if not os.path.exists(out):
        tmp = out + f".{os.getpid()}.tmp"
        subprocess.run(["g++", *FLAGS, "-o", tmp, SRC], check=True)
        os.replace(tmp, out)
    return out


def run_gemv(exe: str, fmt: str, Ns, M: int, K: int, xdt="bf16", ydt="f32", ws_bytes=None, plan=None):
    """Replays one decode launch (the first 16-token block of the call)."""
    Ns = [Ns] if isinstance(Ns, int) else list(Ns)
    if ws_bytes is None:
        ws_bytes = lb.gemv_multi_workspace_bytes(fmt, Ns, M, K)
    plan = plan or lb.gemv_plan(fmt, Ns, M, K, x_dtype=xdt, y_dtype=ydt, workspace_bytes=ws_bytes)
    return _run(exe, plan, fmt, Ns, min(M, 16), K, ydt, ws_bytes), plan


def run_gemm(exe: str, fmt: str, M: int, N: int, K: int, xdt="bf16", ydt="f32", ws_bytes=None, plan=None):
    if ws_bytes is None:
        ws_bytes = lb.gemm_workspace_bytes(fmt, M, N, K)
    plan = plan or lb.gemm_plan(fmt, M, N, K, x_dtype=xdt, y_dtype=ydt, workspace_bytes=ws_bytes)
    return _run(exe, plan, fmt, [N], M, K, ydt, ws_bytes, slots=SLOTS), plan


def _run(exe, plan, fmt, Ns, M, K, ydt, ws_bytes, slots=SLOTS):
    args = [exe, f"kernel={plan['kernel_name']}", f"fmt={lb.FORMATS[fmt]}", f"M={M}", f"K={K}",
            f"y_f16={int(ydt == 'f16')}", f"ws_bytes={ws_bytes}", f"slots={slots}"]
    args += [f"N={n}" for n in Ns]
    for k, v in plan.items():
        if k == "lds_offsets":
            args += [f"lds{i}={x}" for i, x in enumerate(v)]
        elif isinstance(v, int) and k != "kernel":
            args.append(f"{k}={v}")
    r = subprocess.run(args, capture_output=True, text=True)
    return r.returncode, (r.stdout + r.stderr).strip()
