"""ctypes binding of liblowbit.so: argument marshalling only.

Every step of the product runs in the library (host packer, HIP kernels).
There is no Python or CPU fallback: if the library is missing, calls raise.
"""
from __future__ import annotations

import ctypes
import os

import numpy as np

PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(PKG, "liblowbit.so")

FORMATS = {"q1": 1, "tq2": 2, "tq5": 3}
DT_F16, DT_BF16, DT_F32 = 1, 2, 3
GROUP = 128

_lib = None

KERNELS = {0: "none", 1: "gemv_staged", 2: "gemv_split", 3: "gemv_wide", 4: "gemv_tq5", 5: "gemv_tq5_one",
           6: "gemm", 7: "fill_zero", 8: "gemv_kslice"}
OPERANDS = {0: "none", 1: "f16", 2: "bf16", 3: "fp8_fp4", 4: "fp8x3_fp4"}


class Plan(ctypes.Structure):
    """lowbit_plan of include/lowbit.h."""
    _fields_ = [(n, ctypes.c_int) for n in (
        "kernel", "launches", "grid", "threads", "lds_bytes", "token_slots", "operands", "whole_tiles",
        "tiles_per_wave", "waves", "waves_per_tile", "k_ranges", "groups_per_range", "groups_per_pass", "ring",
        "items_per_wg", "x_pieces")] + [("lds_offsets", ctypes.c_int * 3), ("reserved", ctypes.c_int * 4)]

    def as_dict(self) -> dict:
        d = {n: getattr(self, n) for n, _ in self._fields_ if n not in ("lds_offsets", "reserved")}
        d["lds_offsets"] = list(self.lds_offsets)
        d["kernel_name"] = KERNELS.get(self.kernel, "?")
        d["operands_name"] = OPERANDS.get(self.operands, "?")
        return d


class LowbitError(RuntimeError):
    def __init__(self, status: int, msg: str):
        super().__init__(f"lowbit error {status}: {msg}")
        self.status = status


def load() -> ctypes.CDLL:
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"{LIB_PATH} is not built; run `python -m ternary_group_scaled_q1_amd.build`")
    # torch bundles its own HIP runtime and loads it by the unversioned name
    # libamdhip64.so.  If this library were loaded first, its dependency
    # libamdhip64.so.7 would bring in the system runtime and torch would then
    # load a second HIP (and HSA) runtime into the process.  Importing torch
    # first lets the dynamic loader satisfy libamdhip64.so.7 with torch's
    # copy (same SONAME), so the process has exactly one HIP runtime.
    try:
        import torch  # noqa: F401
    except ImportError:
        pass
    lib = ctypes.CDLL(LIB_PATH)
    i64, i32, vp = ctypes.c_int64, ctypes.c_int, ctypes.c_void_p
    sig = {
        "lowbit_abi_version": (i32, []),
        "lowbit_strerror": (ctypes.c_char_p, [i32]),
        "packed_bytes_lowbit": (i64, [i32, i64, i64]),
        "pack_q1_g128": (i32, [vp, vp, i64, i64, vp, i64]),
        "pack_tq2_g128": (i32, [vp, vp, i64, i64, vp, i64]),
        "pack_tq5_g128": (i32, [vp, vp, i64, i64, vp, i64]),
        "unpack_lowbit": (i32, [i32, vp, i64, i64, i64, vp, vp]),
        "import_mlx_q1_g128": (i32, [vp, vp, vp, i32, i64, i64, vp, i64]),
        "gemv_workspace_bytes_lowbit": (i64, [i32, i64, i64, i64]),
        "gemv_lowbit": (i32, [i32, vp, vp, i32, vp, i32, i64, i64, i64, vp, i64, vp]),
        "gemv_multi_workspace_bytes_lowbit": (i64, [i32, i32, vp, i64, i64]),
        "gemv_multi_lowbit": (i32, [i32, i32, vp, vp, vp, i32, vp, i32, i64, i64, vp, i64, vp]),
        "gemm_workspace_bytes_lowbit": (i64, [i32, i64, i64, i64]),
        "gemm_lowbit": (i32, [i32, vp, vp, i32, vp, i32, i64, i64, i64, vp, i64, vp]),
        "gemv_lowbit_noalloc": (i32, [i32, vp, vp, i32, vp, i32, i64, i64, i64, vp]),
        "lowbit_gemv_plan": (i32, [i32, i32, vp, i32, i32, i64, i64, i64, ctypes.POINTER(Plan)]),
        "lowbit_gemm_plan": (i32, [i32, i32, i32, i64, i64, i64, i64, ctypes.POINTER(Plan)]),
    }
    for name, (res, args) in sig.items():
        f = getattr(lib, name)
        f.restype, f.argtypes = res, args
    _lib = lib
    return lib


def _check(status: int):
    if status != 0:
        raise LowbitError(status, load().lowbit_strerror(status).decode())


def _fmt(fmt) -> int:
    if isinstance(fmt, str):
        if fmt not in FORMATS:
            raise ValueError(f"unknown format {fmt!r}")
        return FORMATS[fmt]
    return int(fmt)


def abi_version() -> int:
    return load().lowbit_abi_version()


def strerror(status: int) -> str:
    return load().lowbit_strerror(int(status)).decode()


def packed_bytes(fmt, N: int, K: int) -> int:
    n = load().packed_bytes_lowbit(_fmt(fmt), N, K)
    if n < 0:
        _check(int(n))
    return int(n)


def pack(fmt, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8[N,K], scales uint16[N,K/128] (FP16 bits) -> uint8 blob."""
    codes = np.ascontiguousarray(codes, dtype=np.int8)
    N, K = codes.shape
    scales = np.ascontiguousarray(scales, dtype=np.uint16)
    if scales.shape != (N, K // GROUP):
        raise ValueError("scales must have shape (N, K // 128)")
    f = _fmt(fmt)
    out = np.empty(packed_bytes(f, N, K), dtype=np.uint8)
    fn = {1: load().pack_q1_g128, 2: load().pack_tq2_g128, 3: load().pack_tq5_g128}[f]
    _check(fn(codes.ctypes.data, scales.ctypes.data, N, K, out.ctypes.data, out.size))
    return out


def import_mlx_q1(wq: np.ndarray, scales: np.ndarray, biases: np.ndarray, dtype: str = "f16") -> np.ndarray:
    """MLX affine 1-bit g128 -> Binary g128 blob (see import_mlx_q1_g128).

    wq uint32[N, K/32] (bit k % 32 of word k / 32 is q[n, k]); scales and
    biases [N, K/128] as bit patterns (uint16 for dtype "f16" / "bf16",
    uint32 for "f32") or as float16 / float32 arrays."""
    wq = np.ascontiguousarray(wq, dtype=np.uint32)
    N, W = wq.shape
    K = 32 * W
    sb = {"f16": DT_F16, "bf16": DT_BF16, "f32": DT_F32}[dtype]
    bits = np.uint32 if sb == DT_F32 else np.uint16

    def as_bits(a):
        a = np.ascontiguousarray(a)
        if a.dtype in (np.float16, np.float32):
            a = a.view(bits)
        a = np.ascontiguousarray(a, dtype=bits)
        if a.shape != (N, K // GROUP):
            raise ValueError("scales and biases must have shape (N, K // 128)")
        return a

    scales, biases = as_bits(scales), as_bits(biases)
    out = np.empty(packed_bytes(1, N, K), dtype=np.uint8)
    _check(load().import_mlx_q1_g128(wq.ctypes.data, scales.ctypes.data, biases.ctypes.data, sb, N, K,
                                     out.ctypes.data, out.size))
    return out


def unpack(fmt, blob: np.ndarray, N: int, K: int):
    blob = np.ascontiguousarray(blob, dtype=np.uint8)
    codes = np.empty((N, K), dtype=np.int8)
    scales = np.empty((N, K // GROUP), dtype=np.uint16)
    _check(load().unpack_lowbit(_fmt(fmt), blob.ctypes.data, blob.size, N, K, codes.ctypes.data,
                                scales.ctypes.data))
    return codes, scales


# ------------------------------------------------------------ device calls --
def _torch():
    import torch
    return torch


def _x_dtype(t) -> int:
    torch = _torch()
    if t.dtype == torch.float16:
        return DT_F16
    if t.dtype == torch.bfloat16:
        return DT_BF16
    raise TypeError("x must be float16 or bfloat16")


def _y_dtype(dt) -> int:
    torch = _torch()
    if dt == torch.float32:
        return DT_F32
    if dt == torch.float16:
        return DT_F16
    raise TypeError("out dtype must be float32 or float16")


def _prep(fmt, w, x, N, K, out_dtype, out):
    torch = _torch()
    f = _fmt(fmt)
    if not (w.is_cuda and x.is_cuda):
        raise ValueError("w and x must be device tensors")
    if w.dtype != torch.uint8 or not w.is_contiguous() or w.numel() < packed_bytes(f, N, K):
        raise ValueError("w must be a contiguous uint8 device tensor of packed_bytes(fmt, N, K) bytes")
    if x.dim() == 1:
        x = x.unsqueeze(0)
    if x.dim() != 2 or x.shape[1] != K or not x.is_contiguous():
        raise ValueError("x must be a contiguous (M, K) tensor")
    M = x.shape[0]
    if out is None:
        out = torch.empty((M, N), dtype=out_dtype, device=x.device)
    elif out.shape != (M, N) or not out.is_contiguous() or out.device != x.device:
        raise ValueError("out must be a contiguous (M, N) tensor on x's device")
    return f, x, M, out


def gemv_workspace_bytes(fmt, M: int, N: int, K: int) -> int:
    n = load().gemv_workspace_bytes_lowbit(_fmt(fmt), M, N, K)
    if n < 0:
        _check(int(n))
    return int(n)


def gemv(fmt, w, x, N: int, K: int, out_dtype=None, out=None, workspace=None, stream=None):
    """y[M,N] = x[M,K] @ W^T on the GPU (decode path, M <= 16 preferred).

    workspace: a zero-filled uint8 device tensor of at least
    gemv_workspace_bytes() bytes, reused across calls on one stream (a fresh
    zeroed one is allocated here when None and needed); workspace=False runs
    the path that needs none."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    f, x, M, out = _prep(fmt, w, x, N, K, out_dtype, out)
    if workspace is None:
        need = gemv_workspace_bytes(f, M, N, K)
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device) if need else False
    ws_ptr = workspace.data_ptr() if workspace is not False else None
    ws_n = workspace.numel() if workspace is not False else 0
    s = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
    _check(load().gemv_lowbit(f, w.data_ptr(), x.data_ptr(), _x_dtype(x), out.data_ptr(), _y_dtype(out.dtype),
                              M, N, K, ws_ptr, ws_n, s))
    return out


MAX_FUSED = 4


def _ptr_arrays(ptrs, Ns):
    n = len(ptrs)
    return (ctypes.c_void_p * n)(*ptrs), (ctypes.c_int64 * n)(*Ns)


def gemv_multi_workspace_bytes(fmt, Ns, M: int, K: int) -> int:
    arr = (ctypes.c_int64 * len(Ns))(*Ns)
    n = load().gemv_multi_workspace_bytes_lowbit(_fmt(fmt), len(Ns), arr, M, K)
    if n < 0:
        _check(int(n))
    return int(n)


def gemv_multi(fmt, ws, x, Ns, K: int, out_dtype=None, outs=None, workspace=None, stream=None):
    """[x @ W_i^T for each i] in one fused launch (matrices sharing x and K,
    e.g. q/k/v or gate/up).  ws: list of packed uint8 device tensors; Ns:
    their row counts.  workspace as for gemv()."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    if len(ws) != len(Ns) or not 1 <= len(ws) <= MAX_FUSED:
        raise ValueError(f"need 1..{MAX_FUSED} matrices with one row count each")
    f = _fmt(fmt)
    outs = list(outs) if outs is not None else [None] * len(ws)
    prepped = [_prep(f, w, x, N, K, out_dtype, o) for w, N, o in zip(ws, Ns, outs)]
    xx, M = prepped[0][1], prepped[0][2]
    outs = [p[3] for p in prepped]
    if workspace is None:
        need = gemv_multi_workspace_bytes(f, Ns, M, K)
        workspace = torch.zeros(need, dtype=torch.uint8, device=xx.device) if need else False
    ws_ptr = workspace.data_ptr() if workspace is not False else None
    ws_n = workspace.numel() if workspace is not False else 0
    s = stream if stream is not None else torch.cuda.current_stream(xx.device).cuda_stream
    wa, na = _ptr_arrays([w.data_ptr() for w in ws], Ns)
    ya = (ctypes.c_void_p * len(outs))(*[o.data_ptr() for o in outs])
    _check(load().gemv_multi_lowbit(f, len(ws), wa, na, xx.data_ptr(), _x_dtype(xx), ya, _y_dtype(out_dtype), M, K,
                                    ws_ptr, ws_n, s))
    return outs


def gemv_multi_raw(fmt: int, w_ptrs, Ns, x_ptr: int, x_dtype: int, y_ptrs, y_dtype: int, M: int, K: int,
                   stream_ptr: int, ws_ptr: int = 0, ws_bytes: int = 0) -> None:
    """Pointer-level fused call (no tensor checks) for tight timing loops."""
    wa, na = _ptr_arrays(w_ptrs, Ns)
    ya = (ctypes.c_void_p * len(y_ptrs))(*y_ptrs)
    _check(load().gemv_multi_lowbit(fmt, len(w_ptrs), wa, na, x_ptr, x_dtype, ya, y_dtype, M, K, ws_ptr or None,
                                    ws_bytes, stream_ptr))


def gemm_workspace_bytes(fmt, M: int, N: int, K: int) -> int:
    n = load().gemm_workspace_bytes_lowbit(_fmt(fmt), M, N, K)
    if n < 0:
        _check(int(n))
    return int(n)


def gemm(fmt, w, x, N: int, K: int, out_dtype=None, out=None, workspace=None, stream=None):
    """y[M,N] = x[M,K] @ W^T on the GPU (prefill path).

    workspace: a zero-filled uint8 device tensor of at least
    gemm_workspace_bytes() bytes, reused across calls on one stream (a fresh
    zeroed one is allocated here when None); workspace=False runs whole tiles
    per workgroup, which needs none."""
    torch = _torch()
    out_dtype = out_dtype or torch.float32
    f, x, M, out = _prep(fmt, w, x, N, K, out_dtype, out)
    if workspace is None:
        need = gemm_workspace_bytes(f, M, N, K)
        workspace = torch.zeros(need, dtype=torch.uint8, device=x.device) if need else False
    ws_ptr = workspace.data_ptr() if workspace is not False else None
    ws_n = workspace.numel() if workspace is not False else 0
    s = stream if stream is not None else torch.cuda.current_stream(x.device).cuda_stream
    _check(load().gemm_lowbit(f, w.data_ptr(), x.data_ptr(), _x_dtype(x), out.data_ptr(), _y_dtype(out.dtype),
                              M, N, K, ws_ptr, ws_n, s))
    return out


def gemv_raw(fmt: int, w_ptr: int, x_ptr: int, x_dtype: int, y_ptr: int, y_dtype: int, M: int, N: int, K: int,
             stream_ptr: int, ws_ptr: int = 0, ws_bytes: int = 0) -> None:
    """Pointer-level call (no tensor checks) for tight timing loops."""
    _check(load().gemv_lowbit(fmt, w_ptr, x_ptr, x_dtype, y_ptr, y_dtype, M, N, K, ws_ptr or None, ws_bytes,
                              stream_ptr))


def gemm_raw(fmt: int, w_ptr: int, x_ptr: int, x_dtype: int, y_ptr: int, y_dtype: int, M: int, N: int, K: int,
             stream_ptr: int, ws_ptr: int = 0, ws_bytes: int = 0) -> None:
    _check(load().gemm_lowbit(fmt, w_ptr, x_ptr, x_dtype, y_ptr, y_dtype, M, N, K, ws_ptr or None, ws_bytes,
                              stream_ptr))


def _dt(d) -> int:
    return {"f16": DT_F16, "bf16": DT_BF16, "f32": DT_F32}[d] if isinstance(d, str) else int(d)


def gemv_plan(fmt, Ns, M: int, K: int, x_dtype="bf16", y_dtype="f32", workspace_bytes: int = 0) -> dict:
    """What gemv_lowbit (one row count) or gemv_multi_lowbit (a list) would
    launch with a workspace of workspace_bytes bytes (lowbit_gemv_plan)."""
    Ns = [Ns] if isinstance(Ns, int) else list(Ns)
    arr = (ctypes.c_int64 * len(Ns))(*Ns)
    out = Plan()
    _check(load().lowbit_gemv_plan(_fmt(fmt), len(Ns), arr, _dt(x_dtype), _dt(y_dtype), M, K, workspace_bytes,
                                   ctypes.byref(out)))
    return out.as_dict()


def gemm_plan(fmt, M: int, N: int, K: int, x_dtype="bf16", y_dtype="f32", workspace_bytes: int = 0) -> dict:
    """What gemm_lowbit would launch (lowbit_gemm_plan)."""
    out = Plan()
    _check(load().lowbit_gemm_plan(_fmt(fmt), _dt(x_dtype), _dt(y_dtype), M, N, K, workspace_bytes,
                                   ctypes.byref(out)))
    return out.as_dict()
