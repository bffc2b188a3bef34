"""C-ABI library on the CPU: loads, exports every declared symbol, host packer
parity with the oracle, error paths.  No GPU compute is called here."""
import ctypes
import os
import re

import numpy as np
import pytest

import synth
import ternary_group_scaled_q1_amd as lb
from oracle import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "lowbit.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M)))


def test_library_exports_every_declared_symbol():
    names = declared_functions()
    assert {"pack_q1_g128", "pack_tq2_g128", "pack_tq5_g128", "gemv_lowbit", "gemm_lowbit",
            "unpack_lowbit", "packed_bytes_lowbit"} <= set(names)
    lib = ctypes.CDLL(lb.LIB_PATH)
    for n in names:
        assert hasattr(lib, n), n
    assert lb.abi_version() == 2


def test_strerror_covers_all_codes():
    for st in range(0, -9, -1):
        assert lb.strerror(st) and lb.strerror(st) != "unknown status"
    assert lb.strerror(-100) == "unknown status"


@pytest.mark.parametrize("fmt", ["q1", "tq2", "tq5"])
def test_packed_bytes_closed_form(fmt):
    for N, K in [(0, 0), (1, 128), (7, 640), (151936, 4096), (5120, 17408)]:
        assert lb.packed_bytes(fmt, N, K) == layout.packed_bytes(fmt, N, K)


SHAPES = [(1, 128), (2, 256), (15, 384), (16, 512), (17, 640), (31, 768), (33, 1152), (16, 1280),
          (5, 2048), (40, 896), (48, 17408)]


@pytest.mark.parametrize("fmt", ["q1", "tq2", "tq5"])
def test_pack_matches_oracle_bit_exact(fmt):
    g = np.random.default_rng(2024)
    for N, K in SHAPES:
        codes = synth.codes_binary(g, N, K) if fmt == "q1" else synth.codes_ternary(g, N, K, 0.3)
        sc = g.integers(0, 65536, size=(N, K // 128)).astype(np.uint16)
        blob = lb.pack(fmt, codes, sc)
        assert np.array_equal(blob, layout.pack(fmt, codes, sc)), (fmt, N, K)
        c2, s2 = lb.unpack(fmt, blob, N, K)
        assert np.array_equal(c2, codes) and np.array_equal(s2, sc)


@pytest.mark.parametrize("cfg,mid", [(2, 1), (3, 1), (4, 0), (4, 1)])
def test_pack_matches_oracle_at_workload_shapes(cfg, mid):
    c = synth.CONFIGS[cfg]
    fmt = c["fmt"] if isinstance(c["fmt"], str) else c["fmt"][mid]
    p_zero = c["p_zero"] if not isinstance(c["p_zero"], list) else c["p_zero"][mid]
    N, K = c["shapes"][mid]
    codes, sc = synth.draw_matrix(0, cfg, mid, N, K, p_zero)
    blob = lb.pack(fmt, codes, sc)
    assert np.array_equal(blob, layout.pack(fmt, codes, sc))


def test_pack_error_paths():
    L = lb.load()
    codes = np.ones((2, 128), np.int8)
    sc = np.zeros((2, 1), np.uint16)
    out = np.zeros(lb.packed_bytes("q1", 2, 128), np.uint8)
    p = lambda a: a.ctypes.data
    assert L.pack_q1_g128(p(codes), p(sc), 2, 100, p(out), out.size) == -3       # K % 128
    assert L.pack_q1_g128(p(codes), p(sc), -1, 128, p(out), out.size) == -3      # N < 0
    assert L.pack_q1_g128(p(codes), p(sc), 2, 128, p(out), out.size - 1) == -5   # too small
    assert L.pack_q1_g128(None, p(sc), 2, 128, p(out), out.size) == -1           # NULL
    assert L.packed_bytes_lowbit(9, 2, 128) == -2                                # enum
    z = codes.copy()
    z[1, 5] = 0
    before = out.copy()
    assert L.pack_q1_g128(p(z), p(sc), 2, 128, p(out), out.size) == -4           # 0 is not binary
    assert np.array_equal(out, before)                                          # nothing written
    t = codes.copy()
    t[0, 0] = 2
    out3 = np.zeros(lb.packed_bytes("tq2", 2, 128), np.uint8)
    assert L.pack_tq2_g128(p(t), p(sc), 2, 128, p(out3), out3.size) == -4
    assert L.pack_q1_g128(p(codes), p(sc), 0, 128, None, 0) == 0                 # empty is fine


def test_unpack_rejects_invalid_codes():
    blob = lb.pack("tq2", np.zeros((1, 128), np.int8), np.zeros((1, 1), np.uint16))
    blob[0] = 0xFF  # four code-3 slots
    with pytest.raises(lb.LowbitError) as e:
        lb.unpack("tq2", blob, 1, 128)
    assert e.value.status == -4
    blob5 = lb.pack("tq5", np.zeros((1, 640), np.int8), np.zeros((1, 5), np.uint16))
    blob5[3] = 243
    with pytest.raises(lb.LowbitError):
        lb.unpack("tq5", blob5, 1, 640)
    tail = lb.pack("tq5", np.zeros((1, 128), np.int8), np.zeros((1, 1), np.uint16))
    tail[25] = 121 - 81  # padding trit (offset 25 + 4*26 >= 128) set to -1
    with pytest.raises(lb.LowbitError):
        lb.unpack("tq5", tail, 1, 128)
    with pytest.raises(lb.LowbitError) as e:
        lb.unpack("q1", np.zeros(10, np.uint8), 1, 128)
    assert e.value.status == -5


def test_device_calls_validate_before_launch():
    """Bad arguments are rejected before anything touches a GPU."""
    L = lb.load()
    assert L.gemv_lowbit(7, 16, 16, 1, 16, 3, 1, 1, 128, None, 0, None) == -2            # fmt
    assert L.gemv_lowbit(1, 16, 16, 3, 16, 3, 1, 1, 128, None, 0, None) == -7            # x f32
    assert L.gemv_lowbit(1, 16, 16, 1, 16, 2, 1, 1, 128, None, 0, None) == -7            # y bf16
    assert L.gemv_lowbit(1, 16, 16, 1, 16, 3, 1, 1, 100, None, 0, None) == -3            # K % 128
    assert L.gemv_lowbit(1, None, 16, 1, 16, 3, 1, 1, 128, None, 0, None) == -1          # W NULL
    assert L.gemv_lowbit(1, 8, 16, 1, 16, 3, 1, 1, 128, None, 0, None) == -6             # W misaligned
    assert L.gemv_lowbit(1, 16, 16, 1, 18, 3, 1, 1, 128, None, 0, None) == -6            # Y misaligned (f32)
    assert L.gemv_lowbit(1, None, None, 1, None, 3, 0, 5, 128, None, 0, None) == 0       # M == 0: no-op
    assert L.gemm_lowbit(1, 16, 16, 1, 16, 3, 1, 1, 128, None, -1, None) == -5  # workspace size
    assert L.gemm_lowbit(1, 16, 16, 1, 16, 3, 1, 1, 128, 24, 4096, None) == -6  # workspace misaligned
    assert L.gemm_workspace_bytes_lowbit(1, 512, 17408, 5120) >= 0
    assert L.gemv_lowbit(1, 16, 16, 1, 16, 3, 1, 1, 128, 24, 4096, None) == -6           # workspace misaligned
    assert L.gemv_lowbit(1, 16, 16, 1, 16, 3, 1, 1, 128, None, -1, None) == -5           # workspace size


def test_gemv_workspace_sizes():
    """32 KiB of arrival counters, then the partial sums of at most 16 K
    ranges and 8 MiB (16-token launches); none when fewer than two ranges fit;
    tq5 (it runs on the GEMM kernel) needs none; shape errors reported."""
    L = lb.load()

    def rule(M, N, K):
        m = min(M, 16)
        ks = min(16, (8 << 20) // (m * N * 4), K // 128)
        return 0 if ks < 2 else 32768 + ks * m * N * 4

    for M, N, K in [(1, 5120, 5120), (16, 5120, 5120), (16, 17408, 5120), (16, 151936, 5120), (8, 5120, 17408),
                    (40, 256, 1024), (1, 256, 128)]:
        assert L.gemv_workspace_bytes_lowbit(1, M, N, K) == rule(M, N, K), (M, N, K)
        assert L.gemv_workspace_bytes_lowbit(2, M, N, K) == 0, (M, N, K)
    assert L.gemv_workspace_bytes_lowbit(1, 16, 5120, 5120) == 32768 + 16 * 16 * 5120 * 4
    assert L.gemv_workspace_bytes_lowbit(1, 16, 151936, 5120) == 0
    assert L.gemv_workspace_bytes_lowbit(3, 16, 5120, 17408) == 0
    assert L.gemv_workspace_bytes_lowbit(1, 16, 5120, 100) == -3
    assert L.gemv_workspace_bytes_lowbit(9, 16, 5120, 128) == -2
    assert lb.gemv_workspace_bytes("q1", 16, 5120, 5120) == rule(16, 5120, 5120)


def test_single_hip_runtime_in_process():
    """Loading the library must not bring a second HIP/HSA runtime next to torch's."""
    import subprocess
    import sys
    code = ("import ternary_group_scaled_q1_amd as lb; lb.load(); import torch; "
            "print(sorted({l.split()[-1] for l in open('/proc/self/maps') if 'amdhip64' in l}))")
    out = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True, check=True)
    libs = eval(out.stdout.strip().splitlines()[-1])
    assert len(libs) == 1, libs
