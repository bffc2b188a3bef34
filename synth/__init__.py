"""Seeded synthetic inputs for the low-bit GEMV/GEMM path.

This module only *draws* inputs: sign/trit codes, FP16 group scales and
fp16/bf16 activations, as plain arrays. It contains none of the method's
arithmetic (no packing, no decoding, no products); both the CPU oracle and
the GPU tests/bench take their inputs from here.

Conventions
-----------
* Codes are int8 arrays of shape (N, K) with values in {-1, +1} (binary) or
  {-1, 0, +1} (ternary).  Row n is output feature n, K is the reduction axis.
* Scales are uint16 arrays of shape (N, K // 128) holding IEEE binary16 bit
  patterns, one per 128 consecutive weights of a row.
* Activations are uint16 arrays of shape (M, K) holding fp16 or bf16 bit
  patterns.
* Every float is drawn in float64 and rounded once to its storage type with
  round-to-nearest-even: fp16 by numpy's float64 -> float16 cast, bf16 by
  numpy float64 -> float32 followed by RNE of the float32 to its top 16 bits.
  The rounded values *are* the inputs.
* Every stream is ``numpy.random.default_rng([seed, stream, matrix_id, field])``
  with field 0 = codes, 1 = scales, 2 = activations.
"""
from __future__ import annotations

import numpy as np

FIELD_CODES, FIELD_SCALES, FIELD_X = 0, 1, 2
GROUP = 128


def rng(seed: int, stream: int, matrix_id: int, field: int) -> np.random.Generator:
    return np.random.default_rng([int(seed), int(stream), int(matrix_id), int(field)])


# ---------------------------------------------------------------- codes ----
def codes_binary(g: np.random.Generator, N: int, K: int) -> np.ndarray:
    """i.i.d. Bernoulli(0.5) signs in {-1,+1}; drawn as uniform random bytes."""
    raw = g.integers(0, 256, size=(N * K + 7) // 8, dtype=np.uint8)
    bits = np.unpackbits(raw, bitorder="little")[: N * K].reshape(N, K)
    return (bits.astype(np.int8) * 2 - 1).astype(np.int8)


def codes_ternary(g: np.random.Generator, N: int, K: int, p_zero: float) -> np.ndarray:
    """i.i.d. trits with P(0) = p_zero and P(-1) = P(+1) = (1 - p_zero) / 2.

    p_zero must be a multiple of 1/60 so the draw is exact on a 60-way die.
    """
    n0 = int(round(p_zero * 60))
    assert abs(n0 / 60 - p_zero) < 1e-12 and (60 - n0) % 2 == 0
    die = g.integers(0, 60, size=(N, K), dtype=np.uint8)
    half = (60 - n0) // 2
    out = np.zeros((N, K), dtype=np.int8)
    out[die < half] = -1
    out[die >= half + n0] = 1
    return out


# --------------------------------------------------------------- floats ----
def f64_to_f16_bits(v: np.ndarray) -> np.ndarray:
    return np.asarray(v, dtype=np.float64).astype(np.float16).view(np.uint16)


def f64_to_bf16_bits(v: np.ndarray) -> np.ndarray:
    f = np.asarray(v, dtype=np.float64).astype(np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    return rounded.astype(np.uint16)


def scales_uniform(g: np.random.Generator, N: int, G: int, lo: float, hi: float) -> np.ndarray:
    return f64_to_f16_bits(g.uniform(lo, hi, size=(N, G)))


def scales_absnormal(g: np.random.Generator, N: int, G: int, sigma: float = 0.02,
                     offset: float = 1e-3) -> np.ndarray:
    return f64_to_f16_bits(np.abs(g.normal(0.0, sigma, size=(N, G))) + offset)


def x_normal(g: np.random.Generator, M: int, K: int, dtype: str) -> np.ndarray:
    v = g.normal(0.0, 1.0, size=(M, K))
    if dtype == "f16":
        return f64_to_f16_bits(v)
    if dtype == "bf16":
        return f64_to_bf16_bits(v)
    raise ValueError(dtype)


# ------------------------------------------------- structured test inputs --
def x_small_integers(g: np.random.Generator, M: int, K: int, dtype: str) -> np.ndarray:
    """x in {-2,-1,0,1,2}: exact in fp16 and bf16, so every product and every
    partial sum of the integer-exact case is an exact integer below 2^24."""
    v = g.integers(-2, 3, size=(M, K)).astype(np.float64)
    return f64_to_f16_bits(v) if dtype == "f16" else f64_to_bf16_bits(v)


def scales_const(N: int, G: int, value: float) -> np.ndarray:
    return f64_to_f16_bits(np.full((N, G), value))


def scales_bf16_tie(g: np.random.Generator, N: int, G: int) -> np.ndarray:
    """Scales (1 + 2^-8) * 2^e, e in [-8, -4]: exact in fp16 and exactly halfway
    between two bf16 values, so rounding them to bf16 moves every one by the
    same relative 2^-8 / (1 + 2^-8)."""
    e = g.integers(-8, -3, size=(N, G))
    return f64_to_f16_bits((1.0 + 2.0 ** -8) * np.exp2(e.astype(np.float64)))


def x_f16_tie(g: np.random.Generator, M: int, K: int) -> np.ndarray:
    """fp16 activations +-(1 + 2^-8) * 2^e: exact in fp16, a bf16 half-way tie."""
    e = g.integers(-3, 3, size=(M, K)).astype(np.float64)
    s = np.where(g.integers(0, 2, size=(M, K)) == 1, 1.0, -1.0)
    return f64_to_f16_bits(s * (1.0 + 2.0 ** -8) * np.exp2(e))


def codes_sign_aligned(x_bits_row: np.ndarray, N: int, dtype: str, p_zero: float = 0.0,
                       g: np.random.Generator | None = None) -> np.ndarray:
    """Codes equal to the sign of one activation row (the sign bit of its bit
    pattern), optionally with a random fraction of zeros (ternary)."""
    sign = np.where((x_bits_row.astype(np.uint32) >> 15) & 1, -1, 1).astype(np.int8)
    out = np.tile(sign, (N, 1))
    if p_zero > 0:
        assert g is not None
        out[g.random(out.shape) < p_zero] = 0
    return out


# ------------------------------------------------ workload configurations --
# The workloads the path is measured and checked on, keyed by what they are.
# Shapes are (N, K); ``x`` is the activation dtype; ``p_zero`` is None for
# binary codes; ``stream`` is the workload's fixed id in the seeded draws
# (draw_matrix / draw_x take it), so every draw stays put under any key.
WORKLOADS = {
    "q1_gemv_256x1024": dict(stream=1, name="q1 GEMV 256x1024 M=1 (latency/correctness)", fmt="q1",
            shapes=[(256, 1024)], M=[1], x="f16", y="f32", p_zero=None,
            scales=("uniform", 0.005, 0.05)),
    "q1_decode_8b": dict(stream=2, name="q1 GEMV decode, 8B-class layer shapes, M=1", fmt="q1",
            shapes=[(24576, 4096), (4096, 12288), (151936, 4096)], M=[1], x="f16",
            y="f32", p_zero=None, scales=("absnormal", 0.02, 1e-3)),
    "tq2_decode_27b": dict(stream=3, name="tq2 GEMV, 27B-class shapes, M in {1,4,8}", fmt="tq2",
            shapes=[(34816, 5120), (5120, 17408)], M=[1, 4, 8], x="bf16", y="f32",
            p_zero=0.3, scales=("absnormal", 0.02, 1e-3)),
    "prefill_gemm_512": dict(stream=4, name="prefill GEMM M=512: q1 17408x5120 and tq5 5120x17408", fmt=["q1", "tq5"],
            shapes=[(17408, 5120), (5120, 17408)], M=[512], x="bf16", y="f32",
            p_zero=[None, 1.0 / 3.0], scales=("absnormal", 0.02, 1e-3)),
    "decode_sweep_27b": dict(stream=5, name="~25B-param decode weight sweep (64 blocks + LM head), M in {1,16}",
            fmt=["q1", "tq2"], M=[1, 16], x="bf16", y="f32", p_zero=[None, 0.3],
            scales=("absnormal", 0.02, 1e-3),
            block=[(5120, 5120)] * 4 + [(17408, 5120), (17408, 5120), (5120, 17408)],
            n_blocks=64, head=(151936, 5120)),
}


def draw_matrix(seed: int, stream: int, matrix_id: int, N: int, K: int, p_zero,
                scales=("absnormal", 0.02, 1e-3)):
    """(codes int8[N,K], scales uint16[N,K/128]) for one weight matrix."""
    gc = rng(seed, stream, matrix_id, FIELD_CODES)
    codes = codes_binary(gc, N, K) if p_zero is None else codes_ternary(gc, N, K, p_zero)
    gs = rng(seed, stream, matrix_id, FIELD_SCALES)
    if scales[0] == "uniform":
        s = scales_uniform(gs, N, K // GROUP, scales[1], scales[2])
    else:
        s = scales_absnormal(gs, N, K // GROUP, scales[1], scales[2])
    return codes, s


def draw_x(seed: int, stream: int, matrix_id: int, M: int, K: int, dtype: str) -> np.ndarray:
    return x_normal(rng(seed, stream, matrix_id, FIELD_X), M, K, dtype)
