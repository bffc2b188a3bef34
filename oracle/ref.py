"""The product the low-bit path computes, in float64 (oracle).

TEST INFRASTRUCTURE ONLY: nothing in the product imports this package.

Definition (aberweb.com page, section 4.1: stored bits are mapped to signed
values and multiplied by the FP16 scale of their 128-weight group; ternary
weights are {-1, 0, +1} times the group scale, ksqn.cn page):

    w[n, k] = t[n, k] * s[n, k // 128]
    y[m, n] = sum_k x[m, k] * w[n, k]              (Y = X W^T, nn.Linear order)
    a[m, n] = sum_k |x[m, k] * w[n, k]|

Every product is exact in float64 (at most 11 x 11 significant bits), so the
only rounding is the float64 summation, far below the acceptance bound

    |y_gpu - y| <= 2e-3 * a + 1e-6    for every element.

The dense float64 product uses numpy's matmul as a library step.
"""
from __future__ import annotations

import numpy as np

from . import fp, layout

RTOL = 2e-3
ATOL = 1e-6


def weights_f64(codes: np.ndarray, scales_bits: np.ndarray) -> np.ndarray:
    """w = t * s with s repeated over its 128-weight group (exact)."""
    s = fp.decode_f16(scales_bits)
    return codes.astype(np.float64) * np.repeat(s, layout.GROUP, axis=1)


def product(codes, scales_bits, x_bits, x_dtype: str):
    """(y, a): y = X W^T and a = |X| |W|^T, both float64 of shape (M, N)."""
    w = weights_f64(np.asarray(codes), np.asarray(scales_bits))
    x = fp.decode(np.asarray(x_bits), x_dtype)
    if x.ndim == 1:
        x = x[None, :]
    y = x @ w.T
    a = np.abs(x) @ np.abs(w).T
    return y, a


def product_from_blob(fmt: str, blob, N: int, K: int, x_bits, x_dtype: str, rows=None):
    """Decode the packed blob with the oracle's own unpack, then product()."""
    codes, scales = layout.unpack(fmt, blob, N, K, rows=rows)
    return product(codes, scales, x_bits, x_dtype)


def within_tolerance(y_gpu, y_ref, a_ref):
    """Elementwise acceptance test; returns (ok, worst excess ratio)."""
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    bound = RTOL * np.asarray(a_ref) + ATOL
    err = np.abs(y_gpu - y_ref)
    ok = bool(np.all(err <= bound)) and bool(np.all(np.isfinite(y_gpu)))
    worst = float(np.max(err / bound)) if err.size else 0.0
    return ok, worst
