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
    assert lb.abi_version() == 7


PAGES = ("lnrk.cn page", "ksqn.cn page", "cnblogs.com page", "aberweb.com page")


def declaration_comments():
    """(function name, the comment block nearest before its declaration)."""
    text = open(HEADER).read()
    out = []
    for m in re.finditer(r"^\s*(?:const\s+)?\w+\s*\**\s*(\w+)\s*\(", text, flags=re.M):
        before = text[:m.start()]
        if before.rfind("/*") < 0 or before.rfind("*/") < before.rfind("/*"):
            continue  # inside a comment
        c0 = before.rfind("/*")
        out.append((m.group(1), re.sub(r"\s+", " ", before[c0:])))
    return out


def test_every_declaration_cites_a_page():
    """Each exported call of the C ABI names the passage that defines what it
    does (or, for a variant for callers that cannot allocate, says so)."""
    decls = declaration_comments()
    assert {n for n, _ in decls} == set(declared_functions())
    for name, comment in decls:
        assert any(p in comment for p in PAGES) or "cannot allocate" in comment, name


def test_plan_query_reaches_the_timed_plans():
    """The plan query runs the launchers' own planning code without a GPU
    (256 compute units assumed): the 16-token LM head of the decode sweep
    takes the split kernel with two row tiles per wave and all of K, the
    16-token o launch cuts K, the 16-token q/k/v and gate/up launches take
    the K-sliced kernel (10 waves; 4 and 9 row tiles per workgroup), and one
    token takes the staged kernel."""
    K = 5120
    ws = lb.gemv_multi_workspace_bytes("q1", [5120], 16, K)
    p = lb.gemv_plan("q1", [5120], 16, K, workspace_bytes=ws)
    assert p["kernel_name"] == "gemv_split" and p["k_ranges"] > 1 and p["operands_name"] == "fp8_fp4"
    for fmt, ops in (("q1", "fp8_fp4"), ("tq2", "bf16")):
        for Ns, T in (([5120] * 3, 4), ([17408] * 2, 9)):
            p = lb.gemv_plan(fmt, Ns, 16, K, workspace_bytes=ws)
            assert (p["kernel_name"], p["tiles_per_wave"], p["waves"], p["operands_name"]) == \
                ("gemv_kslice", T, 10, ops), p
    for fmt, ops in (("q1", "fp8_fp4"), ("tq2", "bf16")):
        p = lb.gemv_plan(fmt, 151936, 16, K, workspace_bytes=lb.gemv_workspace_bytes(fmt, 16, 151936, K))
        assert (p["kernel_name"], p["tiles_per_wave"], p["k_ranges"], p["waves"], p["operands_name"]) == \
            ("gemv_split", 2, 1, 8, ops), p
    assert lb.gemv_plan("q1", 5120, 1, K)["kernel_name"] == "gemv_staged"
    assert lb.gemv_plan("q1", 5120, 40, K)["launches"] == 3
    assert lb.gemv_plan("tq5", 34816, 1, K)["kernel_name"] == "gemv_tq5_one"
    assert lb.gemv_plan("q1", 5120, 3, 0)["kernel_name"] == "fill_zero"
    assert lb.gemv_plan("q1", 0, 3, K)["kernel_name"] == "none"
    g = lb.gemm_plan("q1", 512, 17408, K, workspace_bytes=lb.gemm_workspace_bytes("q1", 512, 17408, K))
    assert g["kernel_name"] == "gemm" and g["x_pieces"] == 1 and g["launches"] == 2
    assert lb.gemm_plan("q1", 512, 17408, K)["items_per_wg"] == K // 128  # no workspace: whole tiles
    with pytest.raises(lb.LowbitError):
        lb.gemv_plan("q1", 16, 1, 100)


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


@pytest.mark.parametrize("workload,mid", [("q1_decode_8b", 1), ("tq2_decode_27b", 1), ("prefill_gemm_512", 0),
                                          ("prefill_gemm_512", 1)])
def test_pack_matches_oracle_at_workload_shapes(workload, mid):
    c = synth.WORKLOADS[workload]
    fmt = c["fmt"] if isinstance(c["fmt"], str) else c["fmt"][mid]
    p_zero = c["p_zero"] if not isinstance(c["p_zero"], list) else c["p_zero"][mid]
    N, K = c["shapes"][mid]
    codes, sc = synth.draw_matrix(0, c["stream"], mid, N, K, p_zero)
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
    tq5 (its decode kernels never cut K across workgroups) needs none; shape errors reported."""
    L = lb.load()

    def rule(M, N, K):
        m = min(M, 16)
        ks = min(16, (8 << 20) // (m * N * 4), K // 128)
        return 0 if ks < 2 else 32768 + ks * m * N * 4

    for M, N, K in [(1, 5120, 5120), (16, 5120, 5120), (16, 17408, 5120), (16, 151936, 5120), (8, 5120, 17408),
                    (40, 256, 1024), (1, 256, 128)]:
        assert L.gemv_workspace_bytes_lowbit(1, M, N, K) == rule(M, N, K), (M, N, K)
        assert L.gemv_workspace_bytes_lowbit(2, M, N, K) == rule(M, N, K), (M, N, K)
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


def _mlx_matrix(g, N, K, dtype):
    """Random MLX affine 1-bit matrix whose groups are {-s, +s} (a = 2s, b = -s)."""
    s = synth.scales_absnormal(g, N, K // 128)
    sv = s.view(np.float16).astype(np.float64) * np.where(g.random((N, K // 128)) < 0.1, -1.0, 1.0)
    enc = {"f16": synth.f64_to_f16_bits, "bf16": synth.f64_to_bf16_bits,
           "f32": lambda v: np.asarray(v, dtype=np.float32).view(np.uint32)}[dtype]
    if dtype == "bf16":
        # keep s exact in bf16: round it to 8 significant bits first
        sv = synth.f64_to_bf16_bits(sv).astype(np.uint32)
        sv = (sv << 16).view(np.float32).astype(np.float64)
    wq = g.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    return wq, enc(2 * sv), enc(-sv)


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_import_mlx_matches_oracle(dtype):
    """The library's import equals the oracle's exact Binary g128 form, packed
    by the oracle's own packer, byte for byte."""
    from oracle import mlx
    g = np.random.default_rng(81)
    for N, K in [(1, 128), (17, 640), (40, 1152)]:
        wq, a, b = _mlx_matrix(g, N, K, dtype)
        blob = lb.import_mlx_q1(wq, a, b, dtype)
        codes, s = mlx.to_binary(wq, a, b, dtype)
        assert np.array_equal(blob, layout.pack("q1", codes, s)), (dtype, N, K)


def test_import_mlx_rejections():
    g = np.random.default_rng(82)
    N, K = 4, 256
    wq, a, b = _mlx_matrix(g, N, K, "f32")
    bad = b.copy()
    bad[2, 1] = np.float32(np.float32(bad[2, 1].view(np.float32)) * 2).view(np.uint32)  # a != -2b
    with pytest.raises(lb.LowbitError) as e:
        lb.import_mlx_q1(wq, a, bad, "f32")
    assert e.value.status == -4
    tiny_a = np.full((N, K // 128), np.float32(2 ** -30)).view(np.uint32)
    tiny_b = np.full((N, K // 128), np.float32(-2 ** -31)).view(np.uint32)
    with pytest.raises(lb.LowbitError) as e:
        lb.import_mlx_q1(wq, tiny_a, tiny_b, "f32")   # s below fp16 subnormals
    assert e.value.status == -4
    L = lb.load()
    out = np.zeros(lb.packed_bytes("q1", N, K), dtype=np.uint8)
    assert L.import_mlx_q1_g128(wq.ctypes.data, a.ctypes.data, b.ctypes.data, 9, N, K, out.ctypes.data,
                                out.size) == -2
    assert L.import_mlx_q1_g128(wq.ctypes.data, a.ctypes.data, b.ctypes.data, 3, N, 100, out.ctypes.data,
                                out.size) == -3
    assert L.import_mlx_q1_g128(None, a.ctypes.data, b.ctypes.data, 3, N, K, out.ctypes.data, out.size) == -1
    assert L.import_mlx_q1_g128(wq.ctypes.data, a.ctypes.data, b.ctypes.data, 3, N, K, out.ctypes.data,
                                out.size - 1) == -5
    assert not out.any()  # nothing written on error


def test_gemv_multi_validation():
    """Fused decode GEMV: shapes, counts and pointers are checked for every
    matrix before any launch (no GPU work is reached here)."""
    L = lb.load()
    I64 = ctypes.c_int64
    VP = ctypes.c_void_p
    Ns = (I64 * 3)(5120, 1024, 1024)
    assert L.gemv_multi_workspace_bytes_lowbit(1, 3, Ns, 16, 5120) == lb.gemv_workspace_bytes("q1", 16, 7168, 5120)
    assert L.gemv_multi_workspace_bytes_lowbit(1, 0, Ns, 16, 5120) == -3
    assert L.gemv_multi_workspace_bytes_lowbit(1, 5, Ns, 16, 5120) == -3
    assert L.gemv_multi_workspace_bytes_lowbit(1, 3, None, 16, 5120) == -1
    assert L.gemv_multi_workspace_bytes_lowbit(1, 3, Ns, 16, 100) == -3
    assert L.gemv_multi_workspace_bytes_lowbit(7, 3, Ns, 16, 5120) == -2
    bad = (I64 * 2)(17, -1)
    assert L.gemv_multi_workspace_bytes_lowbit(1, 2, bad, 1, 128) == -3
    # ragged rows round up to whole 16-row tiles in the launch
    assert lb.gemv_multi_workspace_bytes("q1", [17, 33], 16, 5120) == lb.gemv_workspace_bytes("q1", 16, 80, 5120)
    W = (VP * 2)(4096, 8192)
    Y = (VP * 2)(4096, 8192)
    N2 = (I64 * 2)(16, 16)
    args = lambda cnt, w, y, K=128: (1, cnt, w, N2, 4096, 2, y, 1, 1, K, None, 0, None)
    assert L.gemv_multi_lowbit(*args(0, W, Y)) == -3
    assert L.gemv_multi_lowbit(*args(5, W, Y)) == -3
    assert L.gemv_multi_lowbit(*args(2, None, Y)) == -1
    assert L.gemv_multi_lowbit(*args(2, W, None)) == -1
    assert L.gemv_multi_lowbit(*args(2, (VP * 2)(4096, 8200), Y)) == -6       # second W misaligned
    assert L.gemv_multi_lowbit(*args(2, (VP * 2)(4096, None), Y)) == -1       # second W missing
    assert L.gemv_multi_lowbit(*args(2, W, Y, K=100)) == -3
    # M = 0: nothing to do
    assert L.gemv_multi_lowbit(1, 2, W, N2, 4096, 2, Y, 1, 0, 128, None, 0, None) == 0
