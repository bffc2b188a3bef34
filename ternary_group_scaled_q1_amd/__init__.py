"""Packed low-bit (Binary g128 / Ternary g128) GEMV and GEMM for MI355X (gfx950).

Weights stay in their packed form (1 sign bit per weight, or {-1,0,+1} in
2-bit slots or 5 trits per byte, plus one FP16 scale per 128 weights); the
HIP kernels decode them in registers and multiply on the matrix cores.

    import ternary_group_scaled_q1_amd as lb
    blob = lb.pack("q1", codes, scales)            # host, one-time
    y = lb.gemv("q1", torch.from_numpy(blob).cuda(), x, N, K)

The C ABI is declared in include/lowbit.h; this module only marshals
arguments to it (ctypes), with torch providing device memory and streams.
"""
from ._lib import (  # noqa: F401
    DT_BF16, DT_F16, DT_F32, FORMATS, GROUP, LIB_PATH, MAX_FUSED, LowbitError, abi_version, gemm, gemm_plan,
    gemm_raw, gemm_workspace_bytes, gemv, gemv_multi, gemv_multi_raw, gemv_multi_workspace_bytes, gemv_plan,
    gemv_raw, gemv_workspace_bytes, import_mlx_q1, load, pack, packed_bytes, strerror,
    unpack,
)
