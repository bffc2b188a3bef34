"""Exact decoding of 16-bit float bit patterns to float64 (oracle).

TEST INFRASTRUCTURE ONLY: nothing in the product imports this package.

The weight scales are IEEE binary16 ("one FP16 scale per 128 weights": lnrk.cn
page, section on the Binary g128 representation; aberweb.com page, section
4.1).  Activations are fp16 or bf16.  Both decoders follow the IEEE layout
directly: sign bit 15, then a biased exponent, then the fraction; exponent 0
is zero/subnormal and the all-ones exponent is inf/nan.  Every finite value
of either format is exactly representable in float64, so these are exact.
"""
from __future__ import annotations

import numpy as np


def decode_f16(bits) -> np.ndarray:
    """binary16: 1 sign, 5 exponent (bias 15), 10 fraction bits."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 10) & 0x1F
    m = b & 0x3FF
    with np.errstate(over="ignore", invalid="ignore"):
        normal = np.ldexp((1024 + m).astype(np.float64), (e - 25).astype(np.int32))
        sub = np.ldexp(m.astype(np.float64), -24)
        mag = np.where(e == 0, sub, normal)
        mag = np.where(e == 31, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def decode_bf16(bits) -> np.ndarray:
    """bfloat16: 1 sign, 8 exponent (bias 127), 7 fraction bits."""
    b = np.asarray(bits).astype(np.int64) & 0xFFFF
    sign = np.where((b >> 15) & 1, -1.0, 1.0)
    e = (b >> 7) & 0xFF
    m = b & 0x7F
    with np.errstate(over="ignore", invalid="ignore"):
        normal = np.ldexp((128 + m).astype(np.float64), (e - 134).astype(np.int32))
        sub = np.ldexp(m.astype(np.float64), -133)
        mag = np.where(e == 0, sub, normal)
        mag = np.where(e == 255, np.where(m == 0, np.inf, np.nan), mag)
    return sign * mag


def decode(bits, dtype: str) -> np.ndarray:
    if dtype == "f16":
        return decode_f16(bits)
    if dtype == "bf16":
        return decode_bf16(bits)
    if dtype == "f32":
        return np.asarray(bits, dtype=np.uint32).view(np.float32).astype(np.float64)
    raise ValueError(dtype)
