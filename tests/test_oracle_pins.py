"""Pins of the CPU oracle against things other than itself.

Each test checks the oracle against a library routine, an exact rational
brute force, a closed form printed on the pages, a hand-derived golden
example, or an invariant of the mathematics, so that a plausible slip in the
oracle (dropped term, wrong sign, wrong index, transposed operand) fails.
"""
import math
import os
import struct
from fractions import Fraction

import numpy as np
import pytest

import synth
from oracle import fp, layout, ref

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _golden_kv(name):
    out = {}
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            k, v = [s.strip() for s in line.split("=")]
            out[k] = v
    return out


def _golden_rows(name):
    for line in open(os.path.join(GOLDEN, name)):
        line = line.split("#")[0].strip()
        if line:
            yield line.split()


# ------------------------------------------------------------ fp decoding --
def test_decode_f16_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = fp.decode_f16(bits)
    lib = bits.view(np.float16).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    m = ~np.isnan(lib)
    assert np.array_equal(ours[m], lib[m])
    assert np.array_equal(np.signbit(ours[m]), np.signbit(lib[m]))


def test_decode_f16_matches_struct_half():
    for b in (0x0001, 0x03FF, 0x0400, 0x3C00, 0x3C01, 0x7BFF, 0x8001, 0xBC00, 0xFBFF):
        assert fp.decode_f16(np.uint16(b)) == struct.unpack("<e", struct.pack("<H", b))[0]


def test_decode_bf16_all_patterns_match_float32_view():
    bits = np.arange(65536, dtype=np.uint32)
    ours = fp.decode_bf16(bits.astype(np.uint16))
    lib = (bits << 16).astype(np.uint32).view(np.float32).astype(np.float64)
    assert np.array_equal(np.isnan(ours), np.isnan(lib))
    m = ~np.isnan(lib)
    assert np.array_equal(ours[m], lib[m])


# ------------------------------------------------------------------ sizes --
def test_bits_per_weight_closed_forms():
    g = _golden_kv("sizes.txt")
    for N, K in [(1, 128), (7, 256), (16, 4096), (151936, 4096), (5120, 17408)]:
        assert layout.packed_bytes("q1", N, K) * 8 / (N * K) == float(g["q1_bits_per_weight"])
        assert layout.packed_bytes("tq2", N, K) * 8 / (N * K) == float(g["tq2_bits_per_weight"])
    for N, K in [(3, 640), (5120, 5120), (10, 1280)]:
        pa = layout.plane_a_bytes("tq5", N, K)
        assert pa * 8 / (N * K) == float(g["tq5_bits_per_trit"])
        assert math.isclose(layout.packed_bytes("tq5", N, K) * 8 / (N * K),
                            float(g["tq5_bits_per_weight"]), rel_tol=0, abs_tol=1e-15)
    # 3^5 = 243 <= 256 < 3^6: five trits fit a byte, six do not.
    assert 3 ** 5 <= 256 < 3 ** 6
    # ceil(K/5) bytes per row when 640 does not divide K (K = 27*640 + 128)
    assert layout.plane_a_bytes("tq5", 1, 17408) == 3482


def test_8b_model_size_identity_table2():
    g = _golden_kv("sizes.txt")
    params = int(g["fp16_bytes_8b"]) // 2
    assert params % 128 == 0
    # params arranged as rows of one group each; the size depends only on N*K.
    assert layout.packed_bytes("q1", params // 128, 128) == int(g["q1_g128_bytes_8b"])


# ----------------------------------------------------------- value maps ----
def _single_byte_blob(fmt, value):
    # one row whose plane A is the byte `value` repeated; scale 1.0
    if fmt == "q1":
        N, K = 1, 128
    elif fmt == "tq2":
        N, K = 1, 128
    else:
        N, K = 1, 640
    a = layout.plane_a_bytes(fmt, N, K)
    blob = np.concatenate([np.full(a, value, np.uint8),
                           np.array([0x3C00] * (K // 128), np.uint16).view(np.uint8)])
    return blob, N, K


def test_golden_byte_value_maps():
    for row in _golden_rows("codes.txt"):
        fmt, value, want = row[0], int(row[1]), [int(v) for v in row[2:]]
        blob, N, K = _single_byte_blob(fmt, value)
        codes, _ = layout.unpack(fmt, blob, N, K)
        if fmt in ("q1", "tq2"):
            # every byte holds whole fields and all fields of a constant byte are equal
            assert set(codes.ravel().tolist()) == set(want)
        else:
            # every byte of a full tq5 segment holds one trit of each of 5 groups:
            # digit i of byte b is the weight at 128*i + (its offset b in the group)
            for i in range(5):
                assert set(codes[0, 128 * i:128 * (i + 1)].tolist()) == {want[i]}


def test_exhaustive_bytes_valid_counts_and_roundtrip():
    for fmt, n_valid in (("q1", 256), ("tq2", 81), ("tq5", 243)):
        ok = 0
        for v in range(256):
            blob, N, K = _single_byte_blob(fmt, v)
            try:
                codes, sc = layout.unpack(fmt, blob, N, K)
            except layout.FormatError:
                continue
            ok += 1
            assert np.array_equal(layout.pack(fmt, codes, sc), blob)
        assert ok == n_valid, fmt


def test_golden_layout_positions():
    for row in _golden_rows("layout_positions.txt"):
        fmt, N, K, n, k = row[0], int(row[1]), int(row[2]), int(row[3]), int(row[4])
        byte, sub = int(row[6]), int(row[7])
        n_a, k_a = np.int64(n), np.int64(k)
        if fmt == "q1":
            idx = int(layout.q1_bit_index(n_a, k_a, N, K))
            assert (idx // 8, idx % 8) == (byte, sub), row
        elif fmt == "tq2":
            idx = int(layout.tq2_bit_index(n_a, k_a, N, K))
            assert (idx // 8, idx % 8) == (byte, sub), row
        else:
            off, dig = layout.tq5_byte_digit(n_a, k_a, N, K)
            assert (int(off), int(dig)) == (byte, sub), row
        # and the weight really lands there: a single non-default code at (n, k)
        codes = np.full((N, K), -1 if fmt == "q1" else 0, np.int8)
        codes[n, k] = 1
        blob = layout.pack(fmt, codes, np.zeros((N, K // 128), np.uint16))
        base = -1 if fmt == "q1" else 0
        ref_blob = layout.pack(fmt, np.full((N, K), base, np.int8), np.zeros((N, K // 128), np.uint16))
        diff = np.nonzero(blob != ref_blob)[0]
        assert diff.tolist() == [byte], row


def test_golden_scale_positions():
    for row in _golden_rows("scale_positions.txt"):
        fmt, N, K, n, g, want = row[0], int(row[1]), int(row[2]), int(row[3]), int(row[4]), int(row[6])
        assert int(layout.scale_index(fmt, np.int64(n), np.int64(g), N, K)) == want, row
        # and the scale really lands there: one distinct scale at (n, g)
        G = K // 128
        codes = np.full((N, K), -1 if fmt == "q1" else 0, np.int8)
        sc = np.full((N, G), 0x3C00, np.uint16)
        sc[n, g] = 0x4248
        blob = layout.pack(fmt, codes, sc)
        plane_b = blob[layout.plane_a_bytes(fmt, N, K):].view(np.uint16)
        assert np.nonzero(plane_b != 0x3C00)[0].tolist() == [want], row
        _, back = layout.unpack(fmt, blob, N, K)
        assert np.array_equal(back, sc)


SHAPES = [(1, 128), (2, 256), (15, 384), (16, 512), (17, 640), (31, 768), (33, 1152),
          (16, 1280), (5, 2048), (40, 896)]


@pytest.mark.parametrize("fmt", layout.FORMATS)
def test_address_map_is_a_bijection(fmt):
    for N, K in SHAPES:
        nn, kk = np.meshgrid(np.arange(N, dtype=np.int64), np.arange(K, dtype=np.int64), indexing="ij")
        a = layout.plane_a_bytes(fmt, N, K)
        if fmt == "q1":
            idx = layout.q1_bit_index(nn, kk, N, K).ravel()
            assert np.array_equal(np.sort(idx), np.arange(8 * a))
        elif fmt == "tq2":
            idx = layout.tq2_bit_index(nn, kk, N, K).ravel()
            assert np.all(idx % 2 == 0)
            assert np.array_equal(np.sort(idx // 2), np.arange(4 * a))
        else:
            off, dig = layout.tq5_byte_digit(nn, kk, N, K)
            key = (off * 5 + dig).ravel()
            assert np.unique(key).size == N * K and off.min() >= 0 and off.max() < a
            # every byte is used by one row and the row's bytes are contiguous per tile
            assert np.unique(off).size == a
        # plane B: every (row, group) has its own slot, and the scales of one
        # unit (a tile's rows x one chunk of W groups) fill a contiguous range
        G = K // 128
        W = layout.scale_chunk_groups(fmt)
        nn, gg = np.meshgrid(np.arange(N, dtype=np.int64), np.arange(G, dtype=np.int64), indexing="ij")
        si = layout.scale_index(fmt, nn, gg, N, K)
        assert np.array_equal(np.sort(si.ravel()), np.arange(N * G))
        for T in range(-(-N // 16)):
            for c in range(-(-G // W)):
                blk = si[16 * T:16 * T + 16, W * c:W * c + W]
                assert blk.max() - blk.min() + 1 == blk.size


@pytest.mark.parametrize("fmt", layout.FORMATS)
def test_pack_unpack_roundtrip_random(fmt):
    g = np.random.default_rng(1234)
    for N, K in SHAPES:
        codes = synth.codes_binary(g, N, K) if fmt == "q1" else synth.codes_ternary(g, N, K, 0.3)
        sc = g.integers(0, 65536, size=(N, K // 128)).astype(np.uint16)
        blob = layout.pack(fmt, codes, sc)
        assert blob.size == layout.packed_bytes(fmt, N, K)
        c2, s2 = layout.unpack(fmt, blob, N, K)
        assert np.array_equal(c2, codes) and np.array_equal(s2, sc)
        rows = np.array([N - 1, 0])
        c3, s3 = layout.unpack(fmt, blob, N, K, rows=rows)
        assert np.array_equal(c3, codes[rows]) and np.array_equal(s3, sc[rows])


def test_tq5_padding_is_checked():
    codes = np.zeros((1, 128), np.int8)
    blob = layout.pack("tq5", codes, np.zeros((1, 1), np.uint16))
    # byte 25 holds digit 4 at segment offset 25+26*4 = 129 >= 128: padding
    blob[25] = 121 - 81  # digit 4 := 0 (trit -1)
    with pytest.raises(layout.FormatError):
        layout.unpack("tq5", blob, 1, 128)


# --------------------------------------------------------- dot products ----
def _struct_f16(b):
    return struct.unpack("<e", struct.pack("<H", int(b)))[0]


def _struct_bf16(b):
    return struct.unpack("<f", struct.pack("<I", int(b) << 16))[0]


def _brute(codes, sc, x, xdt):
    """Exact rational y and a from the definition, with the library (struct)
    float decoders: y = sum_k x_k * t_k * s_{k//128}."""
    N, K = codes.shape
    M = x.shape[0]
    dec = _struct_f16 if xdt == "f16" else _struct_bf16
    y = [[Fraction(0)] * N for _ in range(M)]
    a = [[Fraction(0)] * N for _ in range(M)]
    for m in range(M):
        xs = [Fraction(dec(v)) for v in x[m]]
        for n in range(N):
            for k in range(K):
                w = int(codes[n, k]) * Fraction(_struct_f16(sc[n, k // 128]))
                y[m][n] += w * xs[k]
                a[m][n] += abs(w * xs[k])
    return y, a


@pytest.mark.parametrize("xdt", ["f16", "bf16"])
def test_product_matches_rational_brute_force(xdt):
    g = np.random.default_rng(7)
    for N, K, M in [(3, 128, 1), (4, 256, 2), (2, 640, 3)]:
        codes = synth.codes_ternary(g, N, K, 0.3)
        # scales: normals, subnormals, negative values
        sc = synth.f64_to_f16_bits(g.normal(0, 0.05, size=(N, K // 128)))
        sc[0, 0] = 0x0003  # subnormal
        x = synth.x_normal(g, M, K, xdt)
        x[0, 1] = 0x0001  # smallest subnormal (f16) / tiny (bf16)
        y, a = ref.product(codes, sc, x, xdt)
        yb, ab = _brute(codes, sc, x, xdt)
        for m in range(M):
            for n in range(N):
                bound = K * 2.0 ** -52 * float(ab[m][n])
                assert abs(Fraction(y[m, n]) - yb[m][n]) <= Fraction(bound)
                assert abs(Fraction(a[m, n]) - ab[m][n]) <= Fraction(bound)


def test_product_fsum_full_row():
    g = np.random.default_rng(9)
    N, K = 3, 17408
    codes = synth.codes_ternary(g, N, K, 0.3)
    sc = synth.scales_absnormal(g, N, K // 128)
    x = synth.x_normal(g, 1, K, "bf16")
    y, a = ref.product(codes, sc, x, "bf16")
    xs = [_struct_bf16(v) for v in x[0]]
    for n in range(N):
        prods = [xs[k] * int(codes[n, k]) * _struct_f16(sc[n, k // 128]) for k in range(K)]
        exact = math.fsum(prods)
        assert abs(y[0, n] - exact) <= K * 2.0 ** -52 * a[0, n]


@pytest.mark.parametrize("fmt", layout.FORMATS)
def test_integer_exact_case(fmt):
    g = np.random.default_rng(11)
    N, K, M = 9, 1280, 2
    codes = synth.codes_binary(g, N, K) if fmt == "q1" else synth.codes_ternary(g, N, K, 0.3)
    sc = synth.scales_const(N, K // 128, 1.0)
    x = synth.x_small_integers(g, M, K, "bf16")
    xi = np.rint(fp.decode_bf16(x)).astype(np.int64)
    want = xi @ codes.astype(np.int64).T
    y, _ = ref.product_from_blob(fmt, layout.pack(fmt, codes, sc), N, K, x, "bf16")
    assert np.array_equal(y, want.astype(np.float64))


def test_invariants():
    g = np.random.default_rng(13)
    N, K = 6, 1280
    t = synth.codes_binary(g, N, K)
    sc = synth.scales_absnormal(g, N, K // 128)
    x = synth.x_normal(g, 2, K, "f16")
    y, a = ref.product(t, sc, x, "f16")
    # negation of every code negates y exactly
    y_neg, _ = ref.product(-t, sc, x, "f16")
    assert np.array_equal(y_neg, -y)
    # doubling every scale doubles y exactly
    s2 = synth.f64_to_f16_bits(2 * fp.decode_f16(sc))
    y2, _ = ref.product(t, s2, x, "f16")
    assert np.array_equal(y2, 2 * y)
    # the same +-1 weights stored as q1, tq2 and tq5 give the same product
    outs = [ref.product_from_blob(f, layout.pack(f, t, sc), N, K, x, "f16")[0] for f in layout.FORMATS]
    assert np.array_equal(outs[0], outs[1]) and np.array_equal(outs[0], outs[2])
    # all-zero ternary weights: y = a = 0
    z = np.zeros_like(t)
    yz, az = ref.product(z, sc, x, "f16")
    assert not yz.any() and not az.any()
    # a >= |y|, and a equals |y| when the codes follow the signs of x
    assert np.all(a >= np.abs(y) - 1e-12 * a)
    ta = synth.codes_sign_aligned(x[0], N, "f16")
    ya, aa = ref.product(ta, sc, x[:1], "f16")
    assert np.allclose(ya, aa, rtol=1e-14, atol=0)


def test_group_axis_is_128_consecutive_weights_of_a_row():
    g = np.random.default_rng(17)
    N, K = 4, 1024
    t = synth.codes_binary(g, N, K)
    x = synth.x_normal(g, 1, K, "bf16")
    for grp in (0, 3, 7):
        sc = np.zeros((N, K // 128), np.uint16)
        sc[:, grp] = 0x3C00
        y, _ = ref.product(t, sc, x, "bf16")
        xv = fp.decode_bf16(x[0])
        want = t[:, 128 * grp:128 * (grp + 1)].astype(np.float64) @ xv[128 * grp:128 * (grp + 1)]
        assert np.array_equal(y[0], want)
    # rows are independent: row n's scales touch only output n
    sc = synth.scales_absnormal(g, N, K // 128)
    y0, _ = ref.product(t, sc, x, "bf16")
    sc2 = sc.copy()
    sc2[2] = synth.f64_to_f16_bits(3 * fp.decode_f16(sc[2]))
    y1, _ = ref.product(t, sc2, x, "bf16")
    assert np.array_equal(np.delete(y0, 2, axis=1), np.delete(y1, 2, axis=1))
    assert not np.array_equal(y0[:, 2], y1[:, 2])


def test_tolerance_rule():
    y_ref = np.array([1.0, -2.0, 0.0])
    a_ref = np.array([10.0, 10.0, 0.0])
    ok, _ = ref.within_tolerance(y_ref + np.array([0.02, -0.02, 1e-6]), y_ref, a_ref)
    assert ok
    ok, _ = ref.within_tolerance(y_ref + np.array([0.0201, 0, 0]), y_ref, a_ref)
    assert not ok
    ok, _ = ref.within_tolerance(np.array([np.nan, -2.0, 0.0]), y_ref, a_ref)
    assert not ok


def test_bf16_rounding_of_scales_breaks_the_bound():
    """The adversarial inputs are sharp: rounding the tie scales to bf16 (a
    precision bug the acceptance rule must catch) is rejected."""
    g = np.random.default_rng(19)
    N, K = 4, 1024
    x = synth.x_normal(g, 1, K, "bf16")
    t = synth.codes_sign_aligned(x[0], N, "bf16")
    sc = synth.scales_bf16_tie(g, N, K // 128)
    y, a = ref.product(t, sc, x, "bf16")
    sv = fp.decode_f16(sc)
    s_bf = fp.decode_bf16(synth.f64_to_bf16_bits(sv))
    bad = fp.decode_bf16(x[0]) @ (t.astype(np.float64) * np.repeat(s_bf, 128, axis=1)).T
    ok, _ = ref.within_tolerance(bad[None, :], y, a)
    assert not ok


# ----------------------------------------------------------- MLX affine --
def _mlx_golden():
    kv = {}
    for line in open(os.path.join(GOLDEN, "mlx_affine.txt")):
        line = line.split("#")[0].strip()
        if line:
            k, v = [s.strip() for s in line.split("=")]
            kv[k] = v
    words = np.array([[int(kv[f"word{i}"], 16) for i in range(4)]], dtype=np.uint32)
    plus = [int(t) for t in kv["plus_at"].split()]
    return kv, words, plus


def test_mlx_golden_example():
    """Hand-worked example: dequantised weights, bit order and the exact
    Binary g128 form."""
    from oracle import mlx
    kv, words, plus = _mlx_golden()
    a = np.array([[int(kv["scale_f16"], 16)]], dtype=np.uint16)
    b = np.array([[int(kv["bias_f16"], 16)]], dtype=np.uint16)
    w = mlx.dequant(words, a, b, "f16")
    want = np.full((1, 128), -0.75)
    want[0, plus] = 0.75
    assert np.array_equal(w, want)
    codes, s = mlx.to_binary(words, a, b, "f16")
    assert s[0, 0] == int(kv["s_f16"], 16)
    assert np.array_equal(codes[0], np.where(want[0] > 0, 1, -1))
    # The Binary g128 weights of the converted group equal MLX's exactly.
    assert np.array_equal(ref.weights_f64(codes, s), w)
    bad = np.array([[int(kv["bad_bias_f16"], 16)]], dtype=np.uint16)
    assert mlx.to_binary(words, a, bad, "f16") is None


def test_mlx_bit_order_single_bits():
    """q[n, k] is bit k % 32 of word k // 32: a word with only bit i set
    gives exactly one q = 1, at k = 32 * word + i (brute force over all)."""
    from oracle import mlx
    for wi in range(4):
        for i in range(32):
            words = np.zeros((1, 4), dtype=np.uint32)
            words[0, wi] = np.uint32(1) << np.uint32(i)
            q = mlx.bits_q(words)
            assert q.sum() == 1 and q[0, 32 * wi + i] == 1


@pytest.mark.parametrize("dtype", ["f16", "bf16", "f32"])
def test_mlx_symmetric_groups_closed_form(dtype):
    """Groups built as a = 2s, b = -s (s an FP16 value representable in the
    dtype) dequantise to exactly +-s, and convert back to s with codes 2q-1."""
    from oracle import mlx
    g = np.random.default_rng(71)
    N, K = 6, 384
    # s with at most 8 significant bits and a modest exponent: exact in all three.
    mant = g.integers(128, 256, size=(N, K // 128))
    ex = g.integers(-12, 4, size=(N, K // 128))
    s = np.ldexp(mant.astype(np.float64), ex - 7) * np.where(g.random((N, K // 128)) < 0.2, -1, 1)
    enc = {"f16": lambda v: v.astype(np.float16).view(np.uint16),
           "bf16": synth.f64_to_bf16_bits,
           "f32": lambda v: v.astype(np.float32).view(np.uint32)}[dtype]
    a, b = enc(2 * s), enc(-s)
    words = g.integers(0, 2 ** 32, size=(N, K // 32), dtype=np.uint64).astype(np.uint32)
    w = mlx.dequant(words, a, b, dtype)
    q = mlx.bits_q(words)
    assert np.array_equal(w, np.where(q == 1, 1.0, -1.0) * np.repeat(s, 128, axis=1))
    codes, s16 = mlx.to_binary(words, a, b, dtype)
    assert np.array_equal(s16, s.astype(np.float16).view(np.uint16))
    assert np.array_equal(ref.weights_f64(codes, s16), w)


def test_mlx_rejections():
    """Groups that are not {-s, +s} with s FP16 have no Binary g128 form:
    a != -2b, s below the FP16 range or with too many bits, non-finite."""
    from oracle import mlx
    words = np.zeros((1, 4), dtype=np.uint32)

    def conv(a, b, dtype):
        return mlx.to_binary(words, np.array([[a]]), np.array([[b]]), dtype)

    f = lambda v: np.uint32(np.array(v, dtype=np.float32).view(np.uint32))
    assert conv(f(2.0), f(-1.0), "f32") is not None
    assert conv(f(2.0), f(-0.5), "f32") is None              # {-0.5, 1.5}
    assert conv(f(2 ** -30), f(-2 ** -31), "f32") is None    # s below fp16 subnormals
    assert conv(f(2.0 + 2 ** -20), f(-1.0 - 2 ** -21), "f32") is None  # 22 significant bits
    assert conv(f(np.inf), f(-np.inf), "f32") is None
    assert conv(f(131072.0), f(-65536.0), "f32") is None    # s beyond fp16 max
    assert conv(f(0.0), f(-0.0), "f32") is not None           # all-zero group: s = +0
