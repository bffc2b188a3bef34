"""GPU parity of every launch the decode benchmark times, at its full shapes,
on every output element.

The 27B-class decode sweep runs, per block, a fused q/k/v launch (3 x
5120x5120), o (5120x5120), a fused gate/up launch (2 x 17408x5120) and down
(5120x17408), then the LM head (151936x5120), with binary (q1) and 2-bit
ternary (tq2) weights at 1 and 16 tokens, bf16 x and fp32 y, all through one
shared caller-owned workspace of the benchmark's size.  Each launch is made
here with the same pointer-level calls (gemv_raw / gemv_multi_raw), the same
workspace size and the same plans, on seeded synthetic weights of the
sweep's distributions, and every output element is compared with the
float64 oracle (in blocks of weight rows).  The 16-token LM head takes the
split kernel with two row tiles per wave and all of K (asserted through the
plan query).
"""
import numpy as np
import pytest

import synth
import ternary_group_scaled_q1_amd as lb
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

K5, K17 = 5120, 17408
LAUNCHES = {  # name: (row counts of the fused matrices, K, matrix ids in the sweep's seeded draws)
    "qkv": ([5120, 5120, 5120], K5, [0, 1, 2]),
    "o": ([5120], K5, [3]),
    "gate_up": ([17408, 17408], K5, [4, 5]),
    "down": ([5120], K17, [6]),
    "lm_head": ([151936], K5, [7]),
}
STREAM = synth.WORKLOADS["decode_sweep_27b"]["stream"]
P_ZERO = {"q1": None, "tq2": 0.3}


def _bench_workspace_bytes(fmt):
    """The benchmark's one workspace: the largest any of its launches asks for."""
    return max(lb.gemv_multi_workspace_bytes(fmt, Ns, m, K) for Ns, K, _ in LAUNCHES.values() for m in (1, 16))


@pytest.fixture(scope="module", params=["q1", "tq2"])
def fmt_ws(request):
    t = gu.torch()
    fmt = request.param
    need = _bench_workspace_bytes(fmt)
    return fmt, need, t.zeros(max(need, 16), dtype=t.uint8, device="cuda")


@pytest.mark.parametrize("launch", list(LAUNCHES))
def test_sweep_launch_every_output(fmt_ws, launch):
    t = gu.torch()
    fmt, ws_bytes, ws = fmt_ws
    Ns, K, mids = LAUNCHES[launch]
    mats = [synth.draw_matrix(1, STREAM, mid, N, K, P_ZERO[fmt]) for mid, N in zip(mids, Ns)]
    blobs = [gu.w_tensor(lb.pack(fmt, c, s)) for c, s in mats]
    # The 1-token and 16-token activations, drawn together; the oracle runs
    # once over all 17 rows.
    x = synth.draw_x(1, STREAM, mids[0], 17, K, "bf16")
    refs = [gu.product_blocked(c, s, x, "bf16") for c, s in mats]
    f = lb.FORMATS[fmt]
    s_ptr = t.cuda.current_stream().cuda_stream
    for M, rows in ((1, slice(0, 1)), (16, slice(1, 17))):
        plan = lb.gemv_plan(fmt, Ns, M, K, workspace_bytes=ws_bytes)
        if launch == "lm_head" and M == 16:
            assert (plan["kernel_name"], plan["tiles_per_wave"], plan["k_ranges"]) == ("gemv_split", 2, 1), plan
        print(f"sweep launch {launch} {fmt} M={M}: plan {plan['kernel_name']} grid {plan['grid']} "
              f"R {plan['tiles_per_wave']} waves {plan['waves']} ranges {plan['k_ranges']}", flush=True)
        xd = gu.x_tensor(np.ascontiguousarray(x[rows]), "bf16")
        ys = [t.full((M, N), float("nan"), dtype=t.float32, device="cuda") for N in Ns]
        if len(Ns) == 1:
            lb.gemv_raw(f, blobs[0].data_ptr(), xd.data_ptr(), lb.DT_BF16, ys[0].data_ptr(), lb.DT_F32, M, Ns[0], K,
                        s_ptr, ws.data_ptr(), ws_bytes)
        else:
            lb.gemv_multi_raw(f, [b.data_ptr() for b in blobs], Ns, xd.data_ptr(), lb.DT_BF16,
                              [y.data_ptr() for y in ys], lb.DT_F32, M, K, s_ptr, ws.data_ptr(), ws_bytes)
        t.cuda.synchronize()
        for i, ((c, s), y, (yr, ar)) in enumerate(zip(mats, ys, refs)):
            gu.check(y.cpu().numpy().astype(np.float64), c, s, x[rows], "bf16",
                     f"sweep {launch} {fmt} M={M} matrix {i}", ref_ya=(yr[rows], ar[rows]))
    assert not ws[:32768].any(), "arrival counters must be left at zero"
