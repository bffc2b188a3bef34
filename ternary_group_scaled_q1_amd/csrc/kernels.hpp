// Launchers shared between the C-ABI front end and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/lowbit.h"

namespace lowbit {

// Matrices that one fused decode launch may cover (they share X and K).
constexpr int kMaxMats = LOWBIT_MAX_FUSED;

struct LaunchArgs {
  int fmt;                // 1 q1, 2 tq2, 3 tq5
  const uint8_t *W;       // packed blob (plane A then plane B)
  const uint16_t *X;      // M x K activations (f16 or bf16 bit patterns)
  void *Y;                // M x N output
  bool x_bf16;            // activation dtype
  bool y_f16;             // output dtype (false: fp32)
  int64_t M, N, K;
  void *ws;          // caller-owned device workspace (may be NULL)
  int64_t ws_bytes;  // its size in bytes
  hipStream_t stream;
  // The matrices of the launch: nmat = 1 and (W, N, Y) for a single product;
  // for a fused decode launch N is the rows of all of them, each rounded up
  // to whole 16-row tiles, and (W, Y) are those of the first.
  int nmat = 1;
  const uint8_t *Ws[kMaxMats] = {};
  void *Ys[kMaxMats] = {};
  int64_t Ns[kMaxMats] = {};
  // When set, the launchers record the plan of the call here and launch
  // nothing (lowbit_gemv_plan / lowbit_gemm_plan).
  lowbit_plan *plan = nullptr;
};

// Starts a plan record: kernel, one launch of `grid` workgroups.
inline lowbit_plan &plan_record(const LaunchArgs &a, int kernel, int grid, int threads, int lds) {
  lowbit_plan &o = *a.plan;
  o = lowbit_plan{};
  o.kernel = kernel;
  o.launches = 1;
  o.grid = grid;
  o.threads = threads;
  o.lds_bytes = lds;
  o.waves = threads / 64;
  o.waves_per_tile = 1;
  o.k_ranges = 1;
  return o;
}

// Fills the matrix list of a single-matrix launch.
inline void single_matrix(LaunchArgs &a) {
  a.nmat = 1;
  a.Ws[0] = a.W;
  a.Ys[0] = a.Y;
  a.Ns[0] = a.N;
}

// Each returns a hipError_t of the launch (hipSuccess when nothing to do).
hipError_t launch_gemv(const LaunchArgs &a);
// GEMV for 9..16 tokens (x operands loaded straight into registers).
hipError_t launch_gemv_wide(const LaunchArgs &a);
// Workspace bytes that let launch_gemv take its fastest path for M tokens.
int64_t gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);
// GEMV on fp8 x fp4 instructions with row blocks x K ranges (bf16 x, M <= 16).
hipError_t launch_gemv_split(const LaunchArgs &a);
// GEMV for 9..16 tokens with waves that split K (no workspace): launches (or
// records the plan of) the product and returns true when the launch suits
// it, with err its hipError_t; returns false otherwise.
bool launch_gemv_kslice(const LaunchArgs &a, hipError_t &err);
int64_t gemv_split_workspace_bytes(int64_t M, int64_t N, int64_t K);
// GEMV for base-3 (tq5) weights, up to 16 tokens.
hipError_t launch_gemv_tq5(const LaunchArgs &a);
hipError_t launch_gemm(const LaunchArgs &a);
// Workspace bytes that let launch_gemm split tiles across workgroups (stream-K).
int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K);
hipError_t launch_fill_zero(void *Y, int64_t bytes, hipStream_t stream);
// Bytes of the library's own decode workspace (gemv_lowbit_noalloc), and the
// call that runs a decode product on it (returns a LOWBIT_* status).
int64_t noalloc_scratch_bytes();
int gemv_noalloc(const LaunchArgs &a);

// Compute units of the current device (cached per device, thread-safe).
int num_cus();
// Workgroups of `kernel` (block `threads`, `lds` dynamic LDS bytes) that one
// compute unit holds at once; cached per (kernel, threads, lds, device).
int resident_blocks(const void *kernel, int threads, int lds);

}  // namespace lowbit
