"""Helpers for the GPU parity tests: upload inputs, call the library through
its binding (C ABI), compare with the oracle computed from the *generated*
codes and scales (never from anything the library produced)."""
import numpy as np

import ternary_group_scaled_q1_amd as lb
from oracle import ref

_TORCH = None


def torch():
    global _TORCH
    if _TORCH is None:
        import torch as t
        if not t.cuda.is_available():
            raise RuntimeError("GPU tests need a visible MI355X")
        _TORCH = t
    return _TORCH


def x_tensor(x_bits: np.ndarray, xdt: str):
    t = torch()
    host = t.from_numpy(np.ascontiguousarray(x_bits).view(np.int16))
    return host.view(t.float16 if xdt == "f16" else t.bfloat16).cuda()


def w_tensor(blob: np.ndarray):
    return torch().from_numpy(np.ascontiguousarray(blob)).cuda()


def run(path: str, fmt: str, blob_dev, x_bits, xdt, ydt, N, K, x_dev=None):
    t = torch()
    x = x_dev if x_dev is not None else x_tensor(x_bits, xdt)
    out_dtype = t.float32 if ydt == "f32" else t.float16
    fn = lb.gemv if path == "gemv" else lb.gemm
    y = fn(fmt, blob_dev, x, N, K, out_dtype=out_dtype)
    t.cuda.synchronize()
    return y.float().cpu().numpy().astype(np.float64)


F16_INF_FROM = 65520.0  # fp32 values at or above this round to inf in fp16 (RNE)


def product_blocked(codes, scales, x_bits, xdt, rows=8192):
    """ref.product over blocks of weight rows (the oracle's own function on
    each block, so the float64 weights of a large matrix are never all in
    memory at once); (y, a) of shape (M, N)."""
    N = codes.shape[0]
    ys, as_ = [], []
    for n0 in range(0, N, rows):
        y, a = ref.product(codes[n0:n0 + rows], scales[n0:n0 + rows], x_bits, xdt)
        ys.append(y)
        as_.append(a)
    return np.concatenate(ys, axis=1), np.concatenate(as_, axis=1)


def check(y_gpu, codes, scales, x_bits, xdt, ctx="", y_f16=False, ref_ya=None):
    """Every element within |y - y_ref| <= 2e-3 a + 1e-6.  With y_f16, an
    element whose fp32 value may have reached the fp16 overflow threshold
    (|y_ref| + 2e-3 a >= 65520) may instead be inf of y_ref's sign."""
    y_ref, a_ref = ref_ya if ref_ya is not None else product_blocked(codes, scales, x_bits, xdt)
    y_gpu = np.asarray(y_gpu, dtype=np.float64)
    if y_f16:
        inf = np.isinf(y_gpu)
        assert np.all(np.sign(y_gpu[inf]) == np.sign(y_ref[inf])), f"{ctx}: fp16 overflow with the wrong sign"
        assert np.all(np.abs(y_ref[inf]) + ref.RTOL * a_ref[inf] >= F16_INF_FROM), f"{ctx}: inf below fp16 overflow"
        y_gpu = np.where(inf, y_ref, y_gpu)
    ok, worst = ref.within_tolerance(y_gpu, y_ref, a_ref)
    if not ok:
        bad = np.argwhere(~(np.abs(y_gpu - y_ref) <= ref.RTOL * a_ref + ref.ATOL))
        m, n = bad[0]
        raise AssertionError(
            f"{ctx}: {len(bad)} elements out of tolerance (worst ratio {worst:.3g}); first at "
            f"(m={m}, n={n}) gpu={y_gpu[m, n]!r} ref={y_ref[m, n]!r} a={a_ref[m, n]!r}")
    return worst
