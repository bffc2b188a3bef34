"""gemv_lowbit_noalloc (the decode product on the library's own device
workspace, for callers that cannot allocate) against gemv_lowbit given a
caller workspace of the same size: the same plans, so bitwise-equal outputs,
and both within the bound of the float64 oracle.  Calls in a row, each on a
smaller problem than the one before, all cutting K across workgroups, so
every call depends on the arrival counters the previous one left at zero.
"""
import numpy as np
import pytest

import synth
import ternary_group_scaled_q1_amd as lb
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SCRATCH_BYTES = (8 << 20) + (32 << 10)  # the library's array: 8 MiB of partial sums + 32 KiB of counters
DT = {"f16": lb.DT_F16, "bf16": lb.DT_BF16, "f32": lb.DT_F32}


def test_noalloc_matches_workspace_entry_point():
    t = gu.torch()
    L = lb.load()
    g = np.random.default_rng(4242)
    s_ptr = t.cuda.current_stream().cuda_stream
    cases = [("q1", 16, 5120, 5120, "bf16", "f32"), ("tq2", 8, 1024, 8192, "bf16", "f16"),
             ("q1", 12, 640, 3072, "f16", "f32")]
    ws = t.zeros(SCRATCH_BYTES, dtype=t.uint8, device="cuda")
    for fmt, M, N, K, xdt, ydt in cases:
        plan = lb.gemv_plan(fmt, N, M, K, x_dtype=xdt, y_dtype=ydt, workspace_bytes=SCRATCH_BYTES)
        print(f"noalloc {fmt} M={M} N={N} K={K} x={xdt} y={ydt}: {plan['kernel_name']} "
              f"ranges {plan['k_ranges']}", flush=True)
        assert plan["k_ranges"] > 1, plan  # every case uses the workspace's counters
        codes = synth.codes_binary(g, N, K) if fmt == "q1" else synth.codes_ternary(g, N, K, 0.3)
        sc = synth.scales_absnormal(g, N, K // 128)
        x = synth.x_normal(g, M, K, xdt)
        w = gu.w_tensor(lb.pack(fmt, codes, sc))
        xd = gu.x_tensor(x, xdt)
        odt = t.float32 if ydt == "f32" else t.float16
        y_na = t.full((M, N), float("nan"), dtype=odt, device="cuda")
        y_ws = t.full((M, N), float("nan"), dtype=odt, device="cuda")
        f, xdc, ydc = lb.FORMATS[fmt], DT[xdt], DT[ydt]
        st = L.gemv_lowbit_noalloc(f, w.data_ptr(), xd.data_ptr(), xdc, y_na.data_ptr(), ydc, M, N, K, s_ptr)
        assert st == 0, lb.strerror(st)
        st = L.gemv_lowbit(f, w.data_ptr(), xd.data_ptr(), xdc, y_ws.data_ptr(), ydc, M, N, K, ws.data_ptr(),
                           SCRATCH_BYTES, s_ptr)
        assert st == 0, lb.strerror(st)
        t.cuda.synchronize()
        assert t.equal(y_na, y_ws), f"noalloc {fmt} M={M} N={N} K={K}"
        gu.check(y_na.float().cpu().numpy().astype(np.float64), codes, sc, x, xdt, f"noalloc {fmt} M={M} N={N}")
    assert not ws[:32768].any()


def test_noalloc_argument_errors():
    """Arguments are checked before anything runs, as for gemv_lowbit."""
    L = lb.load()
    t = gu.torch()
    w = t.zeros(1024, dtype=t.uint8, device="cuda")
    x = t.zeros((1, 128), dtype=t.float16, device="cuda")
    y = t.zeros(64, dtype=t.float32, device="cuda")
    assert L.gemv_lowbit_noalloc(1, w.data_ptr() + 8, x.data_ptr(), 1, y.data_ptr(), 3, 1, 1, 128, None) == -6
    assert L.gemv_lowbit_noalloc(1, w.data_ptr(), x.data_ptr(), 1, y.data_ptr(), 3, 1, 1, 100, None) == -3
    assert L.gemv_lowbit_noalloc(9, w.data_ptr(), x.data_ptr(), 1, y.data_ptr(), 3, 1, 1, 128, None) == -2
    assert L.gemv_lowbit_noalloc(1, w.data_ptr(), x.data_ptr(), 1, None, 3, 1, 1, 128, None) == -1
