"""CPU checks of the kernels' memory addressing and of the host packer under
sanitizers (no GPU).

* The host replica (tests/replica/kernel_addressing.cpp, built with
  AddressSanitizer and UBSan) replays the address arithmetic of every
  workgroup, wave and lane of a launch, for the plan the library's own
  planner picks, against buffers of exactly the sizes the kernels are handed:
  x, packed weights, scales, workspace, outputs and LDS.  Every launch the
  benchmark times and every plan family (staged, 2-D split with one, two or
  four row tiles per wave and 8 or 12 waves, K cut in ranges, x in registers,
  K-sliced waves, base-3 kernels, stream-K GEMM with and without fp8 x
  pieces) is covered,
  plus ragged shapes.  Planted plan mistakes must make it fail.
* The packer's C++ (csrc/pack.cpp) is built with AddressSanitizer + UBSan and
  with ThreadSanitizer and driven on exact-size buffers.
"""
import os
import subprocess
import tempfile

import pytest

import ternary_group_scaled_q1_amd as lb
from tests import addressing as ad

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def exe():
    return ad.build_replica()


def _ok(res):
    (rc, out), plan = res
    assert rc == 0 and out.endswith("ok"), (out[-400:], plan)
    return plan


# Every distinct launch of the timed decode sweep (q/k/v fused, o, gate/up
# fused, down, LM head), both weight formats, 1 and 16 tokens.
SWEEP_LAUNCHES = [([5120] * 3, 5120), ([5120], 5120), ([17408] * 2, 5120), ([5120], 17408), ([151936], 5120)]


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("M", [1, 16])
@pytest.mark.parametrize("Ns,K", SWEEP_LAUNCHES)
def test_sweep_launches_in_bounds(exe, fmt, M, Ns, K):
    _ok(ad.run_gemv(exe, fmt, Ns, M, K))


def test_lm_head_16_tokens_two_tiles_per_wave(exe):
    """The plan of the timed 16-token LM head (split kernel, two row tiles
    per wave, all of K) with every address in bounds, with and without a
    workspace and with fp16 output."""
    for fmt in ("q1", "tq2"):
        for ws in (None, 0):
            for ydt in ("f32", "f16"):
                plan = _ok(ad.run_gemv(exe, fmt, 151936, 16, 5120, ydt=ydt, ws_bytes=ws))
                assert (plan["kernel_name"], plan["tiles_per_wave"], plan["k_ranges"]) == ("gemv_split", 2, 1)


@pytest.mark.parametrize("fmt,Ns,K,Ms,xdt", [
    ("q1", [24576], 4096, [1], "f16"), ("q1", [4096], 12288, [1], "f16"), ("q1", [151936], 4096, [1], "f16"),
    ("tq2", [34816], 5120, [1, 4, 8], "bf16"), ("tq2", [5120], 17408, [1, 4, 8], "bf16"),
    ("tq5", [34816], 5120, [1, 8, 16], "bf16"), ("tq5", [5120], 17408, [1, 8, 16], "bf16"),
    ("q1", [256], 1024, [1], "f16"),
])
def test_workload_decode_launches_in_bounds(exe, fmt, Ns, K, Ms, xdt):
    for M in Ms:
        _ok(ad.run_gemv(exe, fmt, Ns, M, K, xdt=xdt))


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("xdt", ["bf16", "f16"])
def test_kslice_plans_in_bounds(exe, fmt, xdt):
    """The K-sliced 16-token kernel (each wave one chunk of K of all the
    workgroup's row tiles): every plan size it is built for (4, 6, 9 and 12
    tiles per workgroup), K of 8 and 10 chunks, single and fused launches,
    9..16 tokens."""
    seen = set()
    for Ns, K in (([5120] * 3, 5120), ([17408] * 2, 5120), ([12288], 4096), ([24576], 4096), ([40960], 5120),
                  ([4096] * 3, 4096)):
        for M in (9, 13, 16):
            plan = _ok(ad.run_gemv(exe, fmt, Ns, M, K, xdt=xdt))
            assert plan["kernel_name"] == "gemv_kslice", plan
            seen.add(plan["tiles_per_wave"])
    assert seen == {4, 6, 9, 12}, seen


# Ragged and small shapes of the GPU tests: partial row tiles, partial
# chunks, tq5 row tails, fused launches with a zero-row matrix, 2..17 tokens.
SMALL = [(1, 128, 1), (17, 640, 3), (16, 512, 1), (33, 1152, 4), (256, 1024, 1), (300, 2048, 5), (64, 17408, 8),
         (4100, 384, 16), (130, 5120, 17), (48, 4096, 2), (2, 768, 9), (5120, 17408, 4), (700, 12288, 16)]


@pytest.mark.parametrize("fmt", ["q1", "tq2", "tq5"])
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_small_and_ragged_launches_in_bounds(exe, fmt, xdt):
    for N, K, M in SMALL:
        for ws in (None, 0):
            _ok(ad.run_gemv(exe, fmt, N, M, K, xdt=xdt, ws_bytes=ws))
    for M, Ns, K in [(1, [17, 300, 64], 1280), (3, [5120, 1024, 1024], 640), (16, [48, 0, 130], 2048),
                     (9, [16, 16, 16, 16], 17408), (2, [4100], 384)]:
        _ok(ad.run_gemv(exe, fmt, Ns, M, K, xdt=xdt))


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
def test_split_plan_families_in_bounds(exe, fmt):
    """12-wave blocks (34816 rows), four tiles per wave (69632 rows), the
    most K ranges (62 groups), each whole and ragged."""
    seen = set()
    for N, K, M in [(34816, 2048, 8), (34816 - 7, 2048, 16), (69632, 2048, 8), (69632 - 7, 2048, 16),
                    (65536, 2048, 16), (65536 - 7, 2048, 8), (16, 62 * 128, 4), (23, 62 * 128, 16)]:
        for xdt in ("bf16", "f16"):
            p = _ok(ad.run_gemv(exe, fmt, N, M, K, xdt=xdt))
            seen.add((p["kernel_name"], p["waves"], p["tiles_per_wave"], p["k_ranges"] > 1))
    assert ("gemv_split", 12, 1, False) in seen
    assert ("gemv_split", 8, 4, False) in seen
    assert ("gemv_split", 8, 2, False) in seen
    assert ("gemv_split", 8, 1, True) in seen


@pytest.mark.parametrize("fmt,M,N,K", [("q1", 512, 17408, 5120), ("tq5", 512, 5120, 17408), ("tq2", 512, 17408, 5120),
                                       ("q1", 300, 700, 5120), ("tq5", 257, 333, 17408), ("tq2", 129, 1000, 2048),
                                       ("q1", 64, 130, 640), ("tq5", 130, 200, 640), ("q1", 1, 16, 128),
                                       ("tq2", 257, 17, 3200), ("tq5", 64, 130, 17408), ("q1", 200, 33, 896)])
def test_gemm_launches_in_bounds(exe, fmt, M, N, K):
    need = lb.gemm_workspace_bytes(fmt, M, N, K)
    for xdt in ("bf16", "f16"):
        for ws in (need, need - 1, 0):
            _ok(ad.run_gemm(exe, fmt, M, N, K, xdt=xdt, ws_bytes=ws))


def test_replica_catches_planted_mistakes(exe):
    """Plans bent on purpose (on the CPU only) must fail the replica: a
    workspace one partial sum short, a staging pass larger than its LDS
    buffer, a K range too short to cover K, a K-sliced plan with a tile, a
    wave or 1 KB of LDS too few, and a GEMM workspace without room for its
    pieces."""
    K = 5120
    ws = lb.gemv_multi_workspace_bytes("q1", [5120], 16, K)
    plan = lb.gemv_plan("q1", [5120], 16, K, workspace_bytes=ws)
    assert plan["kernel_name"] == "gemv_split" and plan["k_ranges"] > 1
    used = 32768 + plan["k_ranges"] * 16 * 5120 * 4  # counters + the plan's partial sums
    (rc, out), _ = ad.run_gemv(exe, "q1", [5120], 16, K, ws_bytes=used, plan=plan)
    assert rc == 0, out
    (rc, out), _ = ad.run_gemv(exe, "q1", [5120], 16, K, ws_bytes=used - 4, plan=plan)
    assert rc != 0 and "partial sum" in out, out
    bad = dict(plan, groups_per_pass=plan["groups_per_pass"] + 4)
    (rc, out), _ = ad.run_gemv(exe, "q1", [5120], 16, K, ws_bytes=ws, plan=bad)
    assert rc != 0, out
    short = dict(plan, groups_per_range=plan["groups_per_range"] - 4)
    (rc, out), _ = ad.run_gemv(exe, "q1", [5120], 16, K, ws_bytes=ws, plan=short)
    assert rc != 0, out
    ksl = lb.gemv_plan("q1", [5120] * 3, 16, K, workspace_bytes=0)
    assert ksl["kernel_name"] == "gemv_kslice", ksl
    for bent in (dict(ksl, tiles_per_wave=ksl["tiles_per_wave"] - 1), dict(ksl, waves=ksl["waves"] - 1),
                 dict(ksl, lds_bytes=ksl["lds_bytes"] - 1024)):
        (rc, out), _ = ad.run_gemv(exe, "q1", [5120] * 3, 16, K, ws_bytes=0, plan=bent)
        assert rc != 0, out
    one = lb.gemv_plan("tq2", 151936, 16, K, workspace_bytes=0)
    (rc, out), _ = ad.run_gemv(exe, "tq2", 151936, 16, K, ws_bytes=0, plan=dict(one, tiles_per_wave=1))
    assert rc != 0, out
    g = lb.gemm_plan("tq5", 512, 5120, 17408, workspace_bytes=lb.gemm_workspace_bytes("tq5", 512, 5120, 17408))
    (rc, out), _ = ad.run_gemm(exe, "tq5", 512, 5120, 17408, ws_bytes=65536, plan=g)
    assert rc != 0, out


def _build_pack_driver(flags, tag):
    out = os.path.join(tempfile.gettempdir(), f"lowbit_pack_{tag}_{os.getpid()}")
    cmd = ["g++", "-std=c++17", "-O1", "-g", *flags, "-D__host__=", "-D__device__=", "-o", out,
           os.path.join(ROOT, "tests", "replica", "pack_sanitize.cpp"),
           os.path.join(ROOT, "ternary_group_scaled_q1_amd", "csrc", "pack.cpp"), "-lpthread"]
    subprocess.run(cmd, check=True)
    return out


@pytest.mark.parametrize("tag,flags", [("asan", ["-fsanitize=address,undefined", "-fno-sanitize-recover=undefined"]),
                                       ("tsan", ["-fsanitize=thread"])])
def test_packer_under_sanitizers(tag, flags):
    """pack / unpack / MLX import of csrc/pack.cpp on exact-size buffers under
    AddressSanitizer + UBSan, and its worker threads under ThreadSanitizer."""
    exe_path = _build_pack_driver(flags, tag)
    try:
        r = subprocess.run([exe_path], capture_output=True, text=True, timeout=600)
    finally:
        os.remove(exe_path)
    assert r.returncode == 0 and r.stdout.strip().endswith("ok"), (r.stdout + r.stderr)[-2000:]
    assert "ERROR" not in r.stderr and "WARNING: ThreadSanitizer" not in r.stderr, r.stderr[-2000:]


@pytest.mark.gpu
def test_device_plans_in_bounds(exe):
    """The same replay with the plans the planner picks on the GPU (real
    compute-unit count and occupancy, which the CPU run can only assume)."""
    import torch
    assert torch.cuda.is_available()
    for fmt in ("q1", "tq2"):
        for M in (1, 16):
            for Ns, K in SWEEP_LAUNCHES:
                print(f"device plan {fmt} M={M} Ns={Ns} K={K}", flush=True)
                _ok(ad.run_gemv(exe, fmt, Ns, M, K))
    for fmt, Ns, K, Ms, xdt in [("q1", [24576], 4096, [1], "f16"), ("q1", [4096], 12288, [1], "f16"),
                                ("q1", [151936], 4096, [1], "f16"), ("tq2", [34816], 5120, [1, 4, 8], "bf16"),
                                ("tq2", [5120], 17408, [1, 4, 8], "bf16"), ("tq5", [34816], 5120, [1, 8, 16], "bf16"),
                                ("tq5", [5120], 17408, [1, 8, 16], "bf16"), ("q1", [256], 1024, [1], "f16")]:
        for M in Ms:
            _ok(ad.run_gemv(exe, fmt, Ns, M, K, xdt=xdt))
    for N, K, M in SMALL:
        for fmt in ("q1", "tq2", "tq5"):
            _ok(ad.run_gemv(exe, fmt, N, M, K))
    for fmt, M, N, K in [("q1", 512, 17408, 5120), ("tq5", 512, 5120, 17408)]:
        _ok(ad.run_gemm(exe, fmt, M, N, K))
