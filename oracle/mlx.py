"""MLX's grouped affine 1-bit format and its exact Binary g128 form (oracle).

TEST INFRASTRUCTURE ONLY: nothing in the product imports this package.

MLX stores, for every group of 128 weights along K, a scale a and a bias b
next to the bits, so that a weight is a * q + b with q in {0, 1}; storing two
16-bit values per group is what makes its 1-bit package 1.25 bits per weight
against 1.125 for the scale-only format (lnrk.cn page, the MLX packing
paragraph; aberweb.com page, summary section 2).  The bits sit 32 to a
uint32 word along K,
lowest bit first (q[n, k] is bit k % 32 of word k // 32).

A group holds the two values b (q = 0) and a + b (q = 1).  It is a Binary
g128 group, bit 0 -> -s and bit 1 -> +s (lnrk.cn page, Binary g128
section), exactly when b = -s and a + b = +s, i.e. a = -2 b, with s = -b an
FP16 value.  The bits then carry over unchanged: code = 2 q - 1.
"""
from __future__ import annotations

import numpy as np

from . import fp

GROUP = 128


def bits_q(wq: np.ndarray) -> np.ndarray:
    """uint32 [N, K/32] -> q in {0, 1} as uint8 [N, K]."""
    wq = np.asarray(wq, dtype=np.uint32)
    N, W = wq.shape
    shifts = np.arange(32, dtype=np.uint32)
    q = (wq[:, :, None] >> shifts[None, None, :]) & np.uint32(1)
    return q.reshape(N, 32 * W).astype(np.uint8)


def dequant(wq, scales_bits, biases_bits, dtype: str) -> np.ndarray:
    """The weights as MLX defines them, a * q + b per group, in float64
    (exact: q is 0 or 1 and a + b of two 16-bit values fits float64)."""
    q = bits_q(wq).astype(np.float64)
    a = np.repeat(fp.decode(scales_bits, dtype), GROUP, axis=1)
    b = np.repeat(fp.decode(biases_bits, dtype), GROUP, axis=1)
    return a * q + b


def to_binary(wq, scales_bits, biases_bits, dtype: str):
    """(codes int8 [N, K], FP16 scale bits uint16 [N, K/128]) of the same
    matrix, or None when a group is not of the form {-s, +s} with s FP16."""
    a = fp.decode(scales_bits, dtype)
    b = fp.decode(biases_bits, dtype)
    s = -b
    with np.errstate(over="ignore", invalid="ignore"):
        s16 = s.astype(np.float16)
        ok = np.isfinite(a) & np.isfinite(b) & (a == -2.0 * b) & (s16.astype(np.float64) == s)
    if not np.all(ok):
        return None
    codes = bits_q(wq).astype(np.int8) * 2 - 1
    return codes, s16.view(np.uint16)
