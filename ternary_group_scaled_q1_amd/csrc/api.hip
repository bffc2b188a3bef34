// C-ABI entry points: argument validation and dispatch to the HIP launchers.
// Nothing is launched unless every argument is valid; no exception escapes.
#include <hip/hip_runtime.h>

#include "../../include/lowbit.h"
#include "kernels.hpp"
#include "layout.hpp"

using namespace lowbit;

namespace {

// Format, dtype and shape checks of a product (no pointers).
int check_shape(int fmt, int x_dtype, int y_dtype, int64_t M, int64_t N, int64_t K) {
  if (fmt < LOWBIT_Q1_G128 || fmt > LOWBIT_TQ5_G128) return LOWBIT_ERR_ENUM;
  if (x_dtype < LOWBIT_F16 || x_dtype > LOWBIT_F32 || y_dtype < LOWBIT_F16 || y_dtype > LOWBIT_F32)
    return LOWBIT_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || K % kGroup) return LOWBIT_ERR_SHAPE;
  // Index arithmetic inside the kernels is 32-bit per operand; keep every
  // operand below 2^31 elements and every packed blob below 2^31 bytes.
  if (M > (1 << 30) || N > (1 << 30) || K > (1 << 30) || M * K >= (int64_t(1) << 31) ||
      M * N >= (int64_t(1) << 31) || packed_bytes_lowbit(fmt, N, K) >= (int64_t(1) << 31))
    return LOWBIT_ERR_SHAPE;
  if (x_dtype == LOWBIT_F32 || y_dtype == LOWBIT_BF16) return LOWBIT_ERR_DTYPE;
  return LOWBIT_OK;
}

int check_product(int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype, int64_t M,
                  int64_t N, int64_t K) {
  const int st = check_shape(fmt, x_dtype, y_dtype, M, N, K);
  if (st != LOWBIT_OK) return st;
  if (M == 0 || N == 0) return LOWBIT_OK;
  if (!Y) return LOWBIT_ERR_NULL;
  if (K > 0 && (!Wp || !X)) return LOWBIT_ERR_NULL;
  const uintptr_t yw = y_dtype == LOWBIT_F32 ? 4 : 2;
  if ((reinterpret_cast<uintptr_t>(Y) % yw) != 0) return LOWBIT_ERR_ALIGN;
  if (K > 0 && ((reinterpret_cast<uintptr_t>(Wp) & 15) || (reinterpret_cast<uintptr_t>(X) & 15)))
    return LOWBIT_ERR_ALIGN;
  return LOWBIT_OK;
}

int run(bool gemm, int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype, int64_t M, int64_t N,
        int64_t K, void *ws, int64_t ws_bytes, void *stream) {
  LaunchArgs a;
  a.ws = ws;
  a.ws_bytes = ws ? ws_bytes : 0;
  a.fmt = fmt;
  a.W = static_cast<const uint8_t *>(Wp);
  a.X = static_cast<const uint16_t *>(X);
  a.Y = Y;
  a.x_bf16 = x_dtype == LOWBIT_BF16;
  a.y_f16 = y_dtype == LOWBIT_F16;
  a.M = M; a.N = N; a.K = K;
  a.stream = static_cast<hipStream_t>(stream);
  single_matrix(a);
  hipError_t e;
  if (K == 0) {
    e = launch_fill_zero(Y, M * N * (a.y_f16 ? 2 : 4), a.stream);
  } else if (gemm) {
    e = launch_gemm(a);
  } else {
    e = launch_gemv(a);
  }
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_DEVICE;
}

// Rows of a fused launch: each matrix rounded up to whole 16-row tiles.
int64_t launch_rows(int count, const int64_t *Ns) {
  int64_t nv = 0;
  for (int i = 0; i < count; ++i) nv += (Ns[i] + 15) / 16 * 16;
  return nv;
}

int check_multi_shape(int fmt, int count, const int64_t *Ns, int64_t M, int64_t K) {
  if (fmt < LOWBIT_Q1_G128 || fmt > LOWBIT_TQ5_G128) return LOWBIT_ERR_ENUM;
  if (count < 1 || count > kMaxMats) return LOWBIT_ERR_SHAPE;
  if (!Ns) return LOWBIT_ERR_NULL;
  if (M < 0 || K < 0 || K % kGroup) return LOWBIT_ERR_SHAPE;
  for (int i = 0; i < count; ++i)
    if (Ns[i] < 0 || Ns[i] > (1 << 30)) return LOWBIT_ERR_SHAPE;
  if (M * launch_rows(count, Ns) >= (int64_t(1) << 31)) return LOWBIT_ERR_SHAPE;
  return LOWBIT_OK;
}

}  // namespace

extern "C" {

int lowbit_abi_version(void) { return LOWBIT_ABI_VERSION; }

const char *lowbit_strerror(int status) {
  switch (status) {
    case LOWBIT_OK: return "ok";
    case LOWBIT_ERR_NULL: return "a required pointer is NULL";
    case LOWBIT_ERR_ENUM: return "unknown format or dtype";
    case LOWBIT_ERR_SHAPE: return "bad shape (negative size, K not a multiple of 128, or too large)";
    case LOWBIT_ERR_VALUE: return "code or byte outside the format's value set";
    case LOWBIT_ERR_SIZE: return "buffer smaller than required";
    case LOWBIT_ERR_ALIGN: return "misaligned pointer (W and X need 16 bytes, Y its element size)";
    case LOWBIT_ERR_DTYPE: return "unsupported dtype combination (x: f16/bf16, y: f32/f16)";
    case LOWBIT_ERR_DEVICE: return "HIP runtime error";
  }
  return "unknown status";
}

int64_t gemv_workspace_bytes_lowbit(int fmt, int64_t M, int64_t N, int64_t K) {
  if (fmt < LOWBIT_Q1_G128 || fmt > LOWBIT_TQ5_G128) return LOWBIT_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || K % kGroup) return LOWBIT_ERR_SHAPE;
  if (M == 0 || N == 0 || K == 0) return 0;
  return gemv_workspace_bytes(fmt, M, N, K);
}

int gemv_lowbit(int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype, int64_t M, int64_t N,
                int64_t K, void *workspace, int64_t workspace_bytes, void *hip_stream) {
  const int st = check_product(fmt, Wp, X, x_dtype, Y, y_dtype, M, N, K);
  if (st != LOWBIT_OK || M == 0 || N == 0) return st;
  if (workspace_bytes < 0) return LOWBIT_ERR_SIZE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 15)) return LOWBIT_ERR_ALIGN;
  return run(false, fmt, Wp, X, x_dtype, Y, y_dtype, M, N, K, workspace, workspace_bytes, hip_stream);
}

int gemv_lowbit_noalloc(int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype, int64_t M,
                        int64_t N, int64_t K, void *hip_stream) {
  const int st = check_product(fmt, Wp, X, x_dtype, Y, y_dtype, M, N, K);
  if (st != LOWBIT_OK || M == 0 || N == 0) return st;
  if (K == 0) return run(false, fmt, Wp, X, x_dtype, Y, y_dtype, M, N, K, nullptr, 0, hip_stream);
  if (gemv_workspace_bytes(fmt, M < 16 ? M : 16, N, K) > noalloc_scratch_bytes()) return LOWBIT_ERR_SIZE;
  LaunchArgs a;
  a.fmt = fmt;
  a.W = static_cast<const uint8_t *>(Wp);
  a.X = static_cast<const uint16_t *>(X);
  a.Y = Y;
  a.x_bf16 = x_dtype == LOWBIT_BF16;
  a.y_f16 = y_dtype == LOWBIT_F16;
  a.M = M; a.N = N; a.K = K;
  a.ws = nullptr;
  a.ws_bytes = 0;
  a.stream = static_cast<hipStream_t>(hip_stream);
  single_matrix(a);
  return gemv_noalloc(a);
}

int64_t gemm_workspace_bytes_lowbit(int fmt, int64_t M, int64_t N, int64_t K) {
  if (fmt < LOWBIT_Q1_G128 || fmt > LOWBIT_TQ5_G128) return LOWBIT_ERR_ENUM;
  if (M < 0 || N < 0 || K < 0 || K % kGroup) return LOWBIT_ERR_SHAPE;
  if (M == 0 || N == 0 || K == 0) return 0;
  return gemm_workspace_bytes(fmt, M, N, K);
}

int64_t gemv_multi_workspace_bytes_lowbit(int fmt, int count, const int64_t *Ns, int64_t M, int64_t K) {
  const int st = check_multi_shape(fmt, count, Ns, M, K);
  if (st != LOWBIT_OK) return st;
  const int64_t nv = launch_rows(count, Ns);
  if (M == 0 || nv == 0 || K == 0) return 0;
  return gemv_workspace_bytes(fmt, M, nv, K);
}

int gemv_multi_lowbit(int fmt, int count, const void *const *Ws, const int64_t *Ns, const void *X, int x_dtype,
                      void *const *Ys, int y_dtype, int64_t M, int64_t K, void *workspace, int64_t workspace_bytes,
                      void *hip_stream) {
  int st = check_multi_shape(fmt, count, Ns, M, K);
  if (st != LOWBIT_OK) return st;
  if (!Ws || !Ys) return LOWBIT_ERR_NULL;
  for (int i = 0; i < count; ++i) {
    st = check_product(fmt, Ws[i], X, x_dtype, Ys[i], y_dtype, M, Ns[i], K);
    if (st != LOWBIT_OK) return st;
  }
  if (workspace_bytes < 0) return LOWBIT_ERR_SIZE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 15)) return LOWBIT_ERR_ALIGN;
  if (M == 0) return LOWBIT_OK;
  // Matrices without rows take no part.
  LaunchArgs a;
  a.nmat = 0;
  for (int i = 0; i < count; ++i) {
    if (Ns[i] == 0) continue;
    a.Ws[a.nmat] = static_cast<const uint8_t *>(Ws[i]);
    a.Ys[a.nmat] = Ys[i];
    a.Ns[a.nmat] = Ns[i];
    ++a.nmat;
  }
  if (a.nmat == 0) return LOWBIT_OK;
  hipError_t e = hipSuccess;
  if (K == 0) {
    for (int i = 0; i < a.nmat; ++i) {
      st = run(false, fmt, a.Ws[i], X, x_dtype, a.Ys[i], y_dtype, M, a.Ns[i], K, workspace, workspace_bytes,
               hip_stream);
      if (st != LOWBIT_OK) return st;
    }
    return LOWBIT_OK;
  }
  a.ws = workspace;
  a.ws_bytes = workspace ? workspace_bytes : 0;
  a.fmt = fmt;
  a.W = a.Ws[0];
  a.X = static_cast<const uint16_t *>(X);
  a.Y = a.Ys[0];
  a.x_bf16 = x_dtype == LOWBIT_BF16;
  a.y_f16 = y_dtype == LOWBIT_F16;
  a.M = M;
  a.N = launch_rows(a.nmat, a.Ns);
  a.K = K;
  a.stream = static_cast<hipStream_t>(hip_stream);
  e = launch_gemv(a);
  return e == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_DEVICE;
}

int gemm_lowbit(int fmt, const void *Wp, const void *X, int x_dtype, void *Y, int y_dtype, int64_t M, int64_t N,
                int64_t K, void *workspace, int64_t workspace_bytes, void *hip_stream) {
  const int st = check_product(fmt, Wp, X, x_dtype, Y, y_dtype, M, N, K);
  if (st != LOWBIT_OK || M == 0 || N == 0) return st;
  if (workspace_bytes < 0) return LOWBIT_ERR_SIZE;
  if (workspace && (reinterpret_cast<uintptr_t>(workspace) & 15)) return LOWBIT_ERR_ALIGN;
  return run(true, fmt, Wp, X, x_dtype, Y, y_dtype, M, N, K, workspace, workspace_bytes, hip_stream);
}

// Plan queries: the launchers run their planning code with a.plan set and
// record what they would launch instead of launching.  Pointers are
// placeholders that no code dereferences; a non-null workspace stands for a
// caller's buffer of workspace_bytes.
int lowbit_gemv_plan(int fmt, int count, const int64_t *Ns, int x_dtype, int y_dtype, int64_t M, int64_t K,
                     int64_t workspace_bytes, lowbit_plan *out) {
  if (!out) return LOWBIT_ERR_NULL;
  int st = check_multi_shape(fmt, count, Ns, M, K);
  if (st != LOWBIT_OK) return st;
  for (int i = 0; i < count; ++i) {
    st = check_shape(fmt, x_dtype, y_dtype, M, Ns[i], K);
    if (st != LOWBIT_OK) return st;
  }
  if (workspace_bytes < 0) return LOWBIT_ERR_SIZE;
  *out = lowbit_plan{};
  alignas(16) static const uint8_t dummy[16] = {};
  LaunchArgs a;
  a.nmat = 0;
  for (int i = 0; i < count; ++i) {
    if (Ns[i] == 0) continue;
    a.Ws[a.nmat] = dummy;
    a.Ys[a.nmat] = const_cast<uint8_t *>(dummy);
    a.Ns[a.nmat] = Ns[i];
    ++a.nmat;
  }
  if (M == 0 || a.nmat == 0) return LOWBIT_OK;
  a.ws = workspace_bytes > 0 ? const_cast<uint8_t *>(dummy) : nullptr;
  a.ws_bytes = workspace_bytes;
  a.fmt = fmt;
  a.W = a.Ws[0];
  a.X = reinterpret_cast<const uint16_t *>(dummy);
  a.Y = a.Ys[0];
  a.x_bf16 = x_dtype == LOWBIT_BF16;
  a.y_f16 = y_dtype == LOWBIT_F16;
  a.M = M;
  a.N = launch_rows(a.nmat, a.Ns);
  a.K = K;
  a.stream = nullptr;
  a.plan = out;
  if (K == 0) {
    plan_record(a, LOWBIT_KERNEL_FILL_ZERO, 0, 256, 0).launches = a.nmat;
    return LOWBIT_OK;
  }
  return launch_gemv(a) == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_DEVICE;
}

int lowbit_gemm_plan(int fmt, int x_dtype, int y_dtype, int64_t M, int64_t N, int64_t K, int64_t workspace_bytes,
                     lowbit_plan *out) {
  if (!out) return LOWBIT_ERR_NULL;
  const int st = check_shape(fmt, x_dtype, y_dtype, M, N, K);
  if (st != LOWBIT_OK) return st;
  if (workspace_bytes < 0) return LOWBIT_ERR_SIZE;
  *out = lowbit_plan{};
  if (M == 0 || N == 0) return LOWBIT_OK;
  alignas(16) static const uint8_t dummy[16] = {};
  LaunchArgs a;
  a.ws = workspace_bytes > 0 ? const_cast<uint8_t *>(dummy) : nullptr;
  a.ws_bytes = workspace_bytes;
  a.fmt = fmt;
  a.W = dummy;
  a.X = reinterpret_cast<const uint16_t *>(dummy);
  a.Y = const_cast<uint8_t *>(dummy);
  a.x_bf16 = x_dtype == LOWBIT_BF16;
  a.y_f16 = y_dtype == LOWBIT_F16;
  a.M = M; a.N = N; a.K = K;
  a.stream = nullptr;
  a.plan = out;
  single_matrix(a);
  if (K == 0) {
    plan_record(a, LOWBIT_KERNEL_FILL_ZERO, 0, 256, 0);
    return LOWBIT_OK;
  }
  return launch_gemm(a) == hipSuccess ? LOWBIT_OK : LOWBIT_ERR_DEVICE;
}

}  // extern "C"
