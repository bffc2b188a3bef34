"""GPU parity: the HIP path (through the C ABI) against the CPU oracle.

Floating point: every element within |y - y_ref| <= 2e-3 * sum|w x| + 1e-6.
Integer-exact inputs (s = 1, x in {-2..2}): bit-exact.  Inputs are seeded and
synthetic (synth), the oracle works from the generated codes and scales.
"""
import numpy as np
import pytest

import synth
import ternary_group_scaled_q1_amd as lb
from oracle import ref
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

FMTS = ["q1", "tq2", "tq5"]


def _codes(g, fmt, N, K, p_zero=0.3):
    return synth.codes_binary(g, N, K) if fmt == "q1" else synth.codes_ternary(g, N, K, p_zero)


# (N, K, M): ragged row tiles, ragged group chunks, tq5 tails, M up to 17
GEMV_SHAPES = [(1, 128, 1), (17, 640, 3), (16, 512, 1), (33, 1152, 4), (256, 1024, 1), (300, 2048, 5),
               (64, 17408, 8), (4100, 384, 16), (130, 5120, 17), (48, 4096, 2), (2, 768, 9)]
GEMM_SHAPES = [(1, 16, 128), (130, 200, 640), (512, 256, 1280), (257, 17, 3200), (64, 130, 17408),
               (200, 33, 896)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("ydt", ["f32", "f16"])
def test_gemv_small_shapes(fmt, xdt, ydt):
    g = np.random.default_rng(100)
    for N, K, M in GEMV_SHAPES:
        print(f"gemv {fmt} x={xdt} y={ydt} N={N} K={K} M={M}", flush=True)
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, xdt)
        blob = gu.w_tensor(lb.pack(fmt, codes, sc))
        y = gu.run("gemv", fmt, blob, x, xdt, ydt, N, K)
        gu.check(y, codes, sc, x, xdt, f"gemv {fmt} {xdt}->{ydt} N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
@pytest.mark.parametrize("ydt", ["f32", "f16"])
def test_gemm_small_shapes(fmt, xdt, ydt):
    g = np.random.default_rng(200)
    for M, N, K in GEMM_SHAPES:
        print(f"gemm {fmt} x={xdt} y={ydt} M={M} N={N} K={K}", flush=True)
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, xdt)
        blob = gu.w_tensor(lb.pack(fmt, codes, sc))
        y = gu.run("gemm", fmt, blob, x, xdt, ydt, N, K)
        gu.check(y, codes, sc, x, xdt, f"gemm {fmt} {xdt}->{ydt} M={M} N={N} K={K}")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_integer_exact_is_bit_exact(path, fmt, xdt):
    """s = 1 and x in {-2..2}: every partial sum is an integer below 2^24, so
    any fp32 order is exact and the result must equal the oracle bitwise; a
    wrong bit order, plane or code map shows up here."""
    g = np.random.default_rng(300)
    for N, K, M in [(17, 640, 3), (64, 2048, 16), (33, 17408, 1)]:
        print(f"int-exact {path} {fmt} {xdt} N={N} K={K} M={M}", flush=True)
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_const(N, K // 128, 1.0)
        x = synth.x_small_integers(g, M, K, xdt)
        y = gu.run(path, fmt, gu.w_tensor(lb.pack(fmt, codes, sc)), x, xdt, "f32", N, K)
        y_ref, _ = ref.product(codes, sc, x, xdt)
        assert np.array_equal(y, y_ref), f"{path} {fmt} {xdt} N={N} K={K} M={M}"


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("fmt", FMTS)
def test_sign_aligned_ties(path, fmt):
    """y = a exactly (codes follow the sign of x).  Tie scales catch a scale
    rounded to bf16; fp16 tie activations catch x rounded to bf16."""
    g = np.random.default_rng(400)
    N, K = 48, 2048
    for xdt in ("bf16", "f16"):
        x = synth.x_normal(g, 1, K, xdt) if xdt == "bf16" else synth.x_f16_tie(g, 1, K)
        codes = synth.codes_sign_aligned(x[0], N, xdt, p_zero=0.0 if fmt == "q1" else 0.2, g=g)
        sc = synth.scales_bf16_tie(g, N, K // 128)
        y = gu.run(path, fmt, gu.w_tensor(lb.pack(fmt, codes, sc)), x, xdt, "f32", N, K)
        gu.check(y, codes, sc, x, xdt, f"ties {path} {fmt} {xdt}")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
@pytest.mark.parametrize("fmt", FMTS)
def test_deterministic_and_scale_doubling(path, fmt):
    g = np.random.default_rng(500)
    N, K, M = 200, 3200, 4
    codes = _codes(g, fmt, N, K)
    sc = synth.scales_absnormal(g, N, K // 128)
    x = synth.x_normal(g, M, K, "bf16")
    w = gu.w_tensor(lb.pack(fmt, codes, sc))
    y1 = gu.run(path, fmt, w, x, "bf16", "f32", N, K)
    y2 = gu.run(path, fmt, w, x, "bf16", "f32", N, K)
    assert np.array_equal(y1, y2)
    sc2 = synth.f64_to_f16_bits(2 * synth_decode(sc))
    y3 = gu.run(path, fmt, gu.w_tensor(lb.pack(fmt, codes, sc2)), x, "bf16", "f32", N, K)
    assert np.array_equal(y3, 2 * y1)


def synth_decode(sc):
    return sc.view(np.float16).astype(np.float64)


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_formats_agree_on_binary_weights(path):
    g = np.random.default_rng(600)
    N, K, M = 90, 1920, 2
    codes = synth.codes_binary(g, N, K)
    sc = synth.scales_absnormal(g, N, K // 128)
    x = synth.x_normal(g, M, K, "f16")
    for fmt in FMTS:
        y = gu.run(path, fmt, gu.w_tensor(lb.pack(fmt, codes, sc)), x, "f16", "f32", N, K)
        gu.check(y, codes, sc, x, "f16", f"{path} {fmt} on binary weights")


def test_ternary_all_zero_gives_zero():
    N, K = 40, 1280
    codes = np.zeros((N, K), np.int8)
    sc = synth.scales_const(N, K // 128, 0.5)
    x = synth.x_normal(np.random.default_rng(1), 3, K, "bf16")
    for fmt in ("tq2", "tq5"):
        for path in ("gemv", "gemm"):
            y = gu.run(path, fmt, gu.w_tensor(lb.pack(fmt, codes, sc)), x, "bf16", "f32", N, K)
            assert not y.any()


def test_degenerate_sizes():
    t = gu.torch()
    L = lb.load()
    # M == 0 or N == 0: OK, nothing launched or written
    y = t.full((1, 4), 7.0, device="cuda")
    assert L.gemv_lowbit(1, None, None, 1, y.data_ptr(), 3, 0, 4, 128, None, 0, None) == 0
    assert L.gemm_lowbit(1, None, None, 1, y.data_ptr(), 3, 1, 0, 128, None, 0, None) == 0
    t.cuda.synchronize()
    assert (y == 7.0).all()
    # K == 0: the empty sum, Y = 0
    for fn in ("gemv", "gemm"):
        y = t.full((3, 5), 7.0, device="cuda")
        w = t.zeros(16, dtype=t.uint8, device="cuda")
        x = t.zeros((3, 0), dtype=t.float16, device="cuda")
        st = (L.gemv_lowbit(1, w.data_ptr(), w.data_ptr(), 1, y.data_ptr(), 3, 3, 5, 0, None, 0, None) if fn == "gemv"
              else L.gemm_lowbit(1, w.data_ptr(), w.data_ptr(), 1, y.data_ptr(), 3, 3, 5, 0, None, 0, None))
        assert st == 0
        t.cuda.synchronize()
        assert (y == 0).all()
    # misaligned device pointers are refused before launch
    w = t.zeros(1024, dtype=t.uint8, device="cuda")
    x = t.zeros((1, 128), dtype=t.float16, device="cuda")
    y = t.zeros(64, dtype=t.float32, device="cuda")
    assert L.gemv_lowbit(1, w.data_ptr() + 8, x.data_ptr(), 1, y.data_ptr(), 3, 1, 1, 128, None, 0, None) == -6


# ------------------------------------------------ full workload shapes ----
def _full(fmt, N, K, M, xdt, path, workload, mid, p_zero, seed=0):
    """Every output element of one workload-shape call against the oracle
    (computed in blocks of weight rows)."""
    stream = synth.WORKLOADS[workload]["stream"]
    codes, sc = synth.draw_matrix(seed, stream, mid, N, K, p_zero)
    x = synth.draw_x(seed, stream, mid, M, K, xdt)
    w = gu.w_tensor(lb.pack(fmt, codes, sc))
    y = gu.run(path, fmt, w, x, xdt, "f32", N, K)
    gu.check(y, codes, sc, x, xdt, f"{path} {fmt} N={N} K={K} M={M}")


@pytest.mark.parametrize("mid", [0, 1, 2])
def test_workload_q1_decode_8b_shapes(mid):
    N, K = synth.WORKLOADS["q1_decode_8b"]["shapes"][mid]
    print(f"q1 gemv N={N} K={K}", flush=True)
    _full("q1", N, K, 1, "f16", "gemv", "q1_decode_8b", mid, None)


@pytest.mark.parametrize("mid", [0, 1])
@pytest.mark.parametrize("M", [1, 4, 8])
def test_workload_tq2_decode_27b_shapes(mid, M):
    N, K = synth.WORKLOADS["tq2_decode_27b"]["shapes"][mid]
    print(f"tq2 gemv N={N} K={K} M={M}", flush=True)
    _full("tq2", N, K, M, "bf16", "gemv", "tq2_decode_27b", mid, 0.3)


@pytest.mark.parametrize("mid", [0, 1])
def test_workload_prefill_gemm(mid):
    c = synth.WORKLOADS["prefill_gemm_512"]
    N, K = c["shapes"][mid]
    fmt, p0 = c["fmt"][mid], c["p_zero"][mid]
    print(f"{fmt} gemm M=512 N={N} K={K}", flush=True)
    _full(fmt, N, K, 512, "bf16", "gemm", "prefill_gemm_512", mid, p0)


def test_workload_q1_gemv_256x1024_all_outputs():
    c = synth.WORKLOADS["q1_gemv_256x1024"]
    N, K = c["shapes"][0]
    codes, sc = synth.draw_matrix(0, c["stream"], 0, N, K, None, scales=c["scales"])
    x = synth.draw_x(0, c["stream"], 0, 1, K, "f16")
    y = gu.run("gemv", "q1", gu.w_tensor(lb.pack("q1", codes, sc)), x, "f16", "f32", N, K)
    gu.check(y, codes, sc, x, "f16", "q1 gemv 256x1024")


# ------------------------------------------ decode sweep shapes (27B-class) ----
SWEEP_SHAPES = [(5120, 5120), (17408, 5120), (5120, 17408)]


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("shape", SWEEP_SHAPES)
@pytest.mark.parametrize("M", [1, 16])
def test_workload_sweep_shapes(fmt, shape, M):
    N, K = shape
    print(f"{fmt} gemv sweep shape N={N} K={K} M={M}", flush=True)
    _full(fmt, N, K, M, "bf16", "gemv", "decode_sweep_27b", SWEEP_SHAPES.index(shape), None if fmt == "q1" else 0.3)


@pytest.mark.parametrize("mid", [0, 1])
@pytest.mark.parametrize("M", [1, 8, 16])
def test_workload_tq5_decode_27b_shapes(mid, M):
    """Base-3 weights at the 27B-class decode shapes (34816x5120: 8 full
    segments per row; 5120x17408: 27 full segments and a 128-trit tail)."""
    N, K = synth.WORKLOADS["tq2_decode_27b"]["shapes"][mid]
    print(f"tq5 gemv N={N} K={K} M={M}", flush=True)
    _full("tq5", N, K, M, "bf16", "gemv", "tq2_decode_27b", mid, 0.3)




# ------------------------------------------------ bf16 x over a wide range ----
@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_bf16_x_wide_dynamic_range(fmt):
    """The prefill path with bf16 activations spread over 2^-40 .. 2^8 inside
    every 32-value block (exact operands: every element within the bound)."""
    g = np.random.default_rng(310)
    M, N, K = 140, 96, 1408
    codes = _codes(g, fmt, N, K)
    sc = synth.scales_absnormal(g, N, K // 128)
    mag = np.exp2(g.uniform(-40, 8, size=(M, K)))
    xf = mag * np.where(g.random((M, K)) < 0.5, -1.0, 1.0)
    _zero_and_subnormal_groups(g, xf)
    x = synth.f64_to_bf16_bits(xf)
    y = gu.run("gemm", fmt, gu.w_tensor(lb.pack(fmt, codes, sc)), x, "bf16", "f32", N, K)
    gu.check(y, codes, sc, x, "bf16", f"gemm wide range {fmt}")


def _zero_and_subnormal_groups(g, xf):
    """Group 5 all zeros and group 6 all bf16 subnormals (|x| < 2^-126) in
    every token: a 32-value block of the fp8 pieces then has no value to take
    its scale from (scale byte 0, a denormal f32 scale), and must still give
    exact zeros and tiny values."""
    M = xf.shape[0]
    xf[:, 640:768] = 0.0
    xf[:, 768:896] = np.exp2(g.uniform(-133, -127, size=(M, 128))) * np.where(g.random((M, 128)) < 0.5, -1.0, 1.0)


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("M", [1, 2, 3, 8, 16])
def test_bf16_x_wide_dynamic_range(fmt, M):
    """bf16 activations whose magnitudes spread over 2^-40 .. 2^8 inside every
    32-value block, plus whole blocks of tiny values next to large ones: every
    element must stay within the bound."""
    g = np.random.default_rng(300 + M)
    N, K = 96, 2048
    codes = _codes(g, fmt, N, K)
    sc = synth.scales_absnormal(g, N, K // 128)
    mag = np.exp2(g.uniform(-40, 8, size=(M, K)))
    xf = mag * np.where(g.random((M, K)) < 0.5, -1.0, 1.0)
    xf[:, 256:384] *= 2.0 ** -60          # one group of tiny values
    xf[:, 512:520] = 0.0                  # a run of zeros
    _zero_and_subnormal_groups(g, xf)
    x = synth.f64_to_bf16_bits(xf)
    blob = gu.w_tensor(lb.pack(fmt, codes, sc))
    ya = ref.product(codes, sc, x, "bf16")
    for ydt in ("f32", "f16"):
        y = gu.run("gemv", fmt, blob, x, "bf16", ydt, N, K)
        gu.check(y, codes, sc, x, "bf16", f"wide range {fmt} M={M} y={ydt}", y_f16=ydt == "f16", ref_ya=ya)


@pytest.mark.parametrize("N,K", [(96, 2048), (4096 + 48, 12288)])
def test_f16_x_wide_dynamic_range_one_token(N, K):
    """Binary weights with fp16 x at one token run on three fp8 pieces per
    value: activations spread over the whole fp16 range (2^-24 .. 2^15)
    inside every 32-value block, a group of zeros, a group of fp16
    subnormals and a group far below its neighbours must all stay within the
    bound, for fp32 and fp16 output."""
    g = np.random.default_rng(320 + K)
    M = 1
    codes = synth.codes_binary(g, N, K)
    sc = synth.scales_absnormal(g, N, K // 128)
    xf = np.exp2(g.uniform(-24, 15, size=(M, K))) * np.where(g.random((M, K)) < 0.5, -1.0, 1.0)
    xf[:, 640:768] = 0.0                                                   # a group of zeros
    xf[:, 768:896] = np.exp2(g.uniform(-24, -15, size=(M, 128))) * np.where(g.random((M, 128)) < 0.5, -1.0, 1.0)
    xf[:, 1024:1152] = np.exp2(g.uniform(-12, -8, size=(M, 128)))          # far below the groups around it
    x = synth.f64_to_f16_bits(xf)
    plan = lb.gemv_plan("q1", [N], M, K, x_dtype="f16")
    assert plan["operands_name"] == "fp8x3_fp4", plan
    blob = gu.w_tensor(lb.pack("q1", codes, sc))
    ya = ref.product(codes, sc, x, "f16")
    for ydt in ("f32", "f16"):
        y = gu.run("gemv", "q1", blob, x, "f16", ydt, N, K)
        gu.check(y, codes, sc, x, "f16", f"f16 wide range N={N} K={K} y={ydt}", y_f16=ydt == "f16", ref_ya=ya)


@pytest.mark.parametrize("fmt", ["tq2", "tq5"])
@pytest.mark.parametrize("M,K", [(1, 1024), (2, 1024), (4, 1024), (8, 1024), (16, 1024), (130, 1024), (4, 8192),
                                 (16, 8192)])
def test_ternary_outliers_on_zero_weights(fmt, M, K):
    """A huge activation in every 32-value block whose weights are all zero:
    the bound counts only the non-zero products, so the small activations
    next to the outlier must keep their full precision (an activation format
    with one shared exponent per block would lose them)."""
    g = np.random.default_rng(500 + M)
    N = 80
    codes = _codes(g, fmt, N, K)
    codes[:, ::32] = 0
    codes[:, 5::32] = 0
    sc = synth.scales_absnormal(g, N, K // 128)
    xf = g.standard_normal((M, K))
    xf[:, ::32] = np.where(g.random((M, K // 32)) < 0.5, -1.0, 1.0) * 2.0 ** 30
    xf[:, 5::32] *= 2.0 ** -20
    x = synth.f64_to_bf16_bits(xf)
    blob = gu.w_tensor(lb.pack(fmt, codes, sc))
    path = "gemv" if M <= 16 else "gemm"
    y = gu.run(path, fmt, blob, x, "bf16", "f32", N, K)
    gu.check(y, codes, sc, x, "bf16", f"outliers {fmt} M={M}")


def test_shared_workspace_across_shapes():
    """One zero-filled workspace serves calls of different shapes and token
    counts in a row (the split-K counters live at a fixed place and every call
    leaves them zero): every result within the bound, and a second pass over
    the same calls bitwise identical to the first."""
    t = gu.torch()
    g = np.random.default_rng(400)
    cases = [("q1", 17, 130, 5120), ("tq2", 16, 5120, 1024), ("q1", 1, 4100, 2048), ("tq2", 9, 300, 17408),
             ("q1", 16, 1000, 640), ("tq2", 3, 64, 5120)]
    need = max(lb.gemv_workspace_bytes(f, M, N, K) for f, M, N, K in cases)
    assert need > 0
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    data = []
    for fmt, M, N, K in cases:
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, "bf16")
        data.append((fmt, M, N, K, codes, sc, x, gu.w_tensor(lb.pack(fmt, codes, sc)), gu.x_tensor(x, "bf16")))
    outs = []
    for rep in range(2):
        for fmt, M, N, K, codes, sc, x, w, xd in data:
            print(f"shared workspace pass {rep}: {fmt} M={M} N={N} K={K}", flush=True)
            y = lb.gemv(fmt, w, xd, N, K, workspace=ws)
            t.cuda.synchronize()
            yv = y.cpu().numpy().astype(np.float64)
            if rep == 0:
                gu.check(yv, codes, sc, x, "bf16", f"shared ws {fmt} M={M} N={N} K={K}")
                outs.append(yv)
            else:
                assert np.array_equal(yv, outs[len(outs) - len(data) + data.index(next(d for d in data if d[0] == fmt and d[1] == M and d[2] == N and d[3] == K))])
    assert not ws[:32768].any(), "split-K counters must be left at zero"


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
def test_gemv_without_workspace(fmt):
    """With no workspace the decode product takes the paths that need none
    (workgroup-staged, or x straight into registers); same bound."""
    g = np.random.default_rng(500)
    for N, K, M in GEMV_SHAPES + [(5120, 17408, 4), (700, 12288, 16)]:
        print(f"gemv {fmt} no workspace N={N} K={K} M={M}", flush=True)
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, "bf16")
        blob = gu.w_tensor(lb.pack(fmt, codes, sc))
        y = lb.gemv(fmt, blob, gu.x_tensor(x, "bf16"), N, K, workspace=False)
        gu.torch().cuda.synchronize()
        gu.check(y.cpu().numpy().astype(np.float64), codes, sc, x, "bf16", f"no ws {fmt} N={N} K={K} M={M}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemm_without_workspace(fmt):
    """With no workspace every workgroup takes whole tiles; same bound."""
    g = np.random.default_rng(600)
    for M, N, K in GEMM_SHAPES:
        print(f"gemm {fmt} no workspace M={M} N={N} K={K}", flush=True)
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, "bf16")
        blob = gu.w_tensor(lb.pack(fmt, codes, sc))
        y = lb.gemm(fmt, blob, gu.x_tensor(x, "bf16"), N, K, workspace=False)
        gu.torch().cuda.synchronize()
        gu.check(y.cpu().numpy().astype(np.float64), codes, sc, x, "bf16", f"gemm no ws {fmt} M={M} N={N} K={K}")


def test_gemm_shared_workspace_and_split_tiles():
    """One zero-filled workspace across GEMM calls of different shapes (tiles
    split between workgroups are summed through it); a second pass is
    bitwise identical and the counters are left at zero."""
    t = gu.torch()
    g = np.random.default_rng(700)
    cases = [("q1", 300, 700, 5120), ("tq5", 257, 333, 17408), ("tq2", 129, 1000, 2048), ("q1", 64, 130, 640)]
    need = max(lb.gemm_workspace_bytes(f, M, N, K) for f, M, N, K in cases)
    ws = t.zeros(need, dtype=t.uint8, device="cuda")
    data, first = [], []
    for fmt, M, N, K in cases:
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, "bf16")
        data.append((fmt, M, N, K, codes, sc, x, gu.w_tensor(lb.pack(fmt, codes, sc)), gu.x_tensor(x, "bf16")))
    for rep in range(2):
        for idx, (fmt, M, N, K, codes, sc, x, w, xd) in enumerate(data):
            print(f"gemm shared workspace pass {rep}: {fmt} M={M} N={N} K={K}", flush=True)
            y = lb.gemm(fmt, w, xd, N, K, workspace=ws)
            t.cuda.synchronize()
            yv = y.cpu().numpy().astype(np.float64)
            if rep == 0:
                gu.check(yv, codes, sc, x, "bf16", f"gemm shared ws {fmt} M={M} N={N} K={K}")
                first.append(yv)
            else:
                assert np.array_equal(yv, first[idx])
    assert not ws[:65536].any(), "stream-K counters must be left at zero"


def test_gemm_q1_workspace_paths():
    """Binary weights with bf16 x: a full workspace takes the fp8-piece path
    (x converted once per call into the workspace), one byte less takes the
    exact bf16 operands with stream-K, none takes whole tiles; all three meet
    the bound, at several token tiles and a ragged last chunk of groups."""
    t = gu.torch()
    g = np.random.default_rng(720)
    for M, N, K in [(300, 700, 5120), (129, 272, 1408), (16, 130, 640)]:
        codes = _codes(g, "q1", N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, "bf16")
        w, xd = gu.w_tensor(lb.pack("q1", codes, sc)), gu.x_tensor(x, "bf16")
        need = lb.gemm_workspace_bytes("q1", M, N, K)
        for label, ws in [("pieces", t.zeros(need, dtype=t.uint8, device="cuda")),
                          ("stream-K", t.zeros(need - 1, dtype=t.uint8, device="cuda")), ("whole tiles", False)]:
            print(f"q1 gemm {label} M={M} N={N} K={K}", flush=True)
            y = lb.gemm("q1", w, xd, N, K, workspace=ws)
            t.cuda.synchronize()
            gu.check(y.cpu().numpy().astype(np.float64), codes, sc, x, "bf16", f"q1 gemm {label} M={M} N={N} K={K}")


@pytest.mark.parametrize("path", ["gemv", "gemm"])
def test_mlx_affine_import_product(path):
    """An MLX affine 1-bit g128 matrix imported into Binary g128 gives the
    product of MLX's own dequantised weights (scale * q + bias), within the
    bound."""
    from oracle import fp, mlx
    g = np.random.default_rng(600)
    N, K, M = (300, 1280, 3) if path == "gemv" else (200, 640, 130)
    s = synth.scales_absnormal(g, N, K // 128).view(np.float16).astype(np.float64)
    a, b = synth.f64_to_f16_bits(2 * s), synth.f64_to_f16_bits(-s)
    wq = g.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    blob = gu.w_tensor(lb.import_mlx_q1(wq, a, b, "f16"))
    x = synth.x_normal(g, M, K, "bf16")
    y = gu.run(path, "q1", blob, x, "bf16", "f32", N, K)
    w = mlx.dequant(wq, a, b, "f16")
    xf = fp.decode(x, "bf16")
    y_ref, a_ref = xf @ w.T, np.abs(xf) @ np.abs(w).T
    ok, worst = ref.within_tolerance(y, y_ref, a_ref)
    assert ok, f"mlx import {path}: worst ratio {worst}"


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_gemv_multi_fused(fmt, xdt):
    """One fused launch over several matrices sharing x (ragged row counts,
    a matrix without rows, 1..16 tokens): every output within the bound, and
    a second call with a shared workspace bitwise identical to the first."""
    t = gu.torch()
    g = np.random.default_rng(700)
    cases = [(1, [17, 300, 64], 1280), (3, [5120, 1024, 1024], 640), (16, [48, 0, 130], 2048),
             (9, [16, 16, 16, 16], 17408), (2, [4100], 384), (20, [33, 64], 1024)]
    for M, Ns, K in cases:
        print(f"multi {fmt} {xdt} M={M} Ns={Ns} K={K}", flush=True)
        mats = []
        for N in Ns:
            codes = _codes(g, fmt, N, K)
            sc = synth.scales_absnormal(g, N, K // 128)
            mats.append((codes, sc, gu.w_tensor(lb.pack(fmt, codes, sc))))
        x = synth.x_normal(g, M, K, xdt)
        xt = gu.x_tensor(x, xdt)
        need = lb.gemv_multi_workspace_bytes(fmt, Ns, M, K)
        ws = t.zeros(max(need, 16), dtype=t.uint8, device="cuda")
        for ydt in ("f32", "f16"):
            odt = t.float32 if ydt == "f32" else t.float16
            ys = lb.gemv_multi(fmt, [m[2] for m in mats], xt, Ns, K, out_dtype=odt, workspace=ws)
            ys2 = lb.gemv_multi(fmt, [m[2] for m in mats], xt, Ns, K, out_dtype=odt, workspace=ws)
            t.cuda.synchronize()
            for i, ((codes, sc, _), y, y2) in enumerate(zip(mats, ys, ys2)):
                assert t.equal(y, y2), (fmt, M, Ns, i)
                if Ns[i] == 0:
                    continue
                yn = y.float().cpu().numpy().astype(np.float64)
                gu.check(yn, codes, sc, x, xdt, f"multi {fmt} {xdt} M={M} Ns={Ns} mat {i} y={ydt}", y_f16=ydt == "f16")
        # no workspace: the paths that need none
        ys = lb.gemv_multi(fmt, [m[2] for m in mats], xt, Ns, K, workspace=False)
        t.cuda.synchronize()
        for i, ((codes, sc, _), y) in enumerate(zip(mats, ys)):
            if Ns[i]:
                gu.check(y.cpu().numpy().astype(np.float64), codes, sc, x, xdt, f"multi no-ws {fmt} mat {i}")


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("M", [8, 16])
@pytest.mark.parametrize("xdt", ["bf16", "f16"])
def test_split_twelve_wave_row_blocks(fmt, M, xdt):
    """34816 rows (2176 row tiles, more than 8 but at most 12 per CU): the
    2-D split takes workgroups of 12 waves with one tile each (fp8 pieces
    for q1 with bf16 x, exact operands otherwise); also a ragged last tile of
    the same tile count (the general load path)."""
    g = np.random.default_rng(930 + M)
    K = 2048
    for N in (34816, 34816 - 7):
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, xdt)
        print(f"12-wave split {fmt} {xdt} M={M} N={N}", flush=True)
        y = gu.run("gemv", fmt, gu.w_tensor(lb.pack(fmt, codes, sc)), x, xdt, "f32", N, K)
        gu.check(y, codes, sc, x, xdt, f"12-wave split {fmt} {xdt} M={M} N={N}")


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("M", [8, 16])
def test_split_tall_matrix_four_tiles_per_wave(fmt, M):
    """69632 rows: the 2-D split's row blocks of one or two tiles per wave
    exceed the CUs, so it takes four (and cuts K); also a ragged last tile
    of the same height (the general load path)."""
    g = np.random.default_rng(910 + M)
    K = 2048
    for N in (69632, 69632 - 7):
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, "bf16")
        y = gu.run("gemv", fmt, gu.w_tensor(lb.pack(fmt, codes, sc)), x, "bf16", "f32", N, K)
        gu.check(y, codes, sc, x, "bf16", f"tall split {fmt} M={M} N={N}")


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("M", [4, 16])
def test_split_most_k_ranges_reused_workspace(fmt, M):
    """One row block and 62 groups: the 2-D split cuts K into 16 ranges of 4
    groups and a last one of 2 (ragged chunk, general load path), so the
    last workgroup adds two batches of 8 ranges.  The same workspace serves
    three calls in a row (fp32 out, fp16 out, fp32 again): the arrival
    counters must be back at zero after each, and the repeat is bit-equal."""
    t = gu.torch()
    g = np.random.default_rng(950 + M)
    K = 62 * 128
    for N in (16, 23):
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, "bf16")
        blob = gu.w_tensor(lb.pack(fmt, codes, sc))
        xd = gu.x_tensor(x, "bf16")
        need = lb.gemv_workspace_bytes(fmt, M, N, K)
        ws = t.zeros(max(need, 1), dtype=t.uint8, device="cuda")
        ys = []
        for odt in (t.float32, t.float16, t.float32):
            print(f"most K ranges {fmt} M={M} N={N} out={odt}", flush=True)
            y = lb.gemv(fmt, blob, xd, N, K, out_dtype=odt, workspace=ws)
            t.cuda.synchronize()
            ys.append(y.float().cpu().numpy().astype(np.float64))
        for i, y in enumerate(ys):
            gu.check(y, codes, sc, x, "bf16", f"most K ranges {fmt} M={M} N={N} call {i}")
        assert np.array_equal(ys[0], ys[2])
        if need:
            assert int(ws[:4 * ((N + 15) // 16)].view(t.int32).abs().sum()) == 0  # counters reset


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("xdt", ["bf16", "f16"])
def test_kslice_every_output(fmt, xdt):
    """The K-sliced kernel (9..16 tokens; each wave one chunk of K of all
    the workgroup's row tiles, x in registers): every plan size it is built
    for (4, 6, 9, 12 tiles per workgroup), K of 8 and 10 chunks, single and
    fused launches, 9, 13 and 16 tokens; every output element against the
    oracle, fp32 and fp16 y, and a repeat bitwise equal (no workspace)."""
    t = gu.torch()
    g = np.random.default_rng(1200)
    cases = [(13, [12288], 4096), (16, [24576], 4096), (9, [17408, 17408], 5120), (16, [40960], 5120),
             (16, [4096, 4096, 4096], 4096)]
    seen = set()
    for M, Ns, K in cases:
        plan = lb.gemv_plan(fmt, Ns, M, K, x_dtype=xdt, workspace_bytes=0)
        assert plan["kernel_name"] == "gemv_kslice", plan
        seen.add(plan["tiles_per_wave"])
        print(f"kslice {fmt} {xdt} M={M} Ns={Ns} K={K} T={plan['tiles_per_wave']}", flush=True)
        mats = []
        for N in Ns:
            codes = _codes(g, fmt, N, K)
            sc = synth.scales_absnormal(g, N, K // 128)
            mats.append((codes, sc, gu.w_tensor(lb.pack(fmt, codes, sc))))
        x = synth.x_normal(g, M, K, xdt)
        xt = gu.x_tensor(x, xdt)
        refs = [gu.product_blocked(codes, sc, x, xdt) for codes, sc, _ in mats]
        for ydt in ("f32", "f16"):
            odt = t.float32 if ydt == "f32" else t.float16
            ys = lb.gemv_multi(fmt, [m[2] for m in mats], xt, Ns, K, out_dtype=odt)
            ys2 = lb.gemv_multi(fmt, [m[2] for m in mats], xt, Ns, K, out_dtype=odt)
            t.cuda.synchronize()
            for i, ((codes, sc, _), y, y2, ref) in enumerate(zip(mats, ys, ys2, refs)):
                assert t.equal(y, y2), (fmt, M, Ns, i)
                gu.check(y.cpu().numpy().astype(np.float64), codes, sc, x, xdt,
                         f"kslice {fmt} {xdt} {ydt} M={M} matrix {i}", y_f16=ydt == "f16", ref_ya=ref)
    assert seen == {4, 6, 9, 12}, seen


@pytest.mark.parametrize("fmt", ["q1", "tq2"])
@pytest.mark.parametrize("xdt", ["bf16", "f16"])
def test_split_two_tiles_per_wave_every_output(fmt, xdt):
    """4096 row tiles (N = 65536, and 65529 with a ragged last tile): the
    2-D split's one-tile row blocks exceed the CUs, so it takes two row
    tiles per wave and all of K, the plan of the 16-token LM head; 8 and 16
    tokens, bf16 and fp16 x (fp8 pieces and exact operands), every output
    element against the oracle."""
    t = gu.torch()
    g = np.random.default_rng(1300)
    K = 2048
    for N in (65536, 65529):
        codes = _codes(g, fmt, N, K)
        sc = synth.scales_absnormal(g, N, K // 128)
        w = gu.w_tensor(lb.pack(fmt, codes, sc))
        for M in (8, 16):
            plan = lb.gemv_plan(fmt, N, M, K, x_dtype=xdt, workspace_bytes=lb.gemv_workspace_bytes(fmt, M, N, K))
            assert (plan["kernel_name"], plan["tiles_per_wave"], plan["k_ranges"]) == ("gemv_split", 2, 1), plan
            print(f"split R=2 {fmt} {xdt} N={N} M={M}", flush=True)
            x = synth.x_normal(g, M, K, xdt)
            ws = t.zeros(max(lb.gemv_workspace_bytes(fmt, M, N, K), 16), dtype=t.uint8, device="cuda")
            y = lb.gemv(fmt, w, gu.x_tensor(x, xdt), N, K, workspace=ws)
            t.cuda.synchronize()
            gu.check(y.cpu().numpy().astype(np.float64), codes, sc, x, xdt, f"split R=2 {fmt} {xdt} N={N} M={M}")
