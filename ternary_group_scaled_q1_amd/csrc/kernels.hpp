// Launchers shared between the C-ABI front end and the kernel translation units.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

struct LaunchArgs {
  int fmt;                // 1 q1, 2 tq2, 3 tq5
  const uint8_t *W;       // packed blob (plane A then plane B)
  const uint16_t *X;      // M x K activations (f16 or bf16 bit patterns)
  void *Y;                // M x N output
  bool x_bf16;            // activation dtype
  bool y_f16;             // output dtype (false: fp32)
  int64_t M, N, K;
  hipStream_t stream;
};

// Each returns a hipError_t of the launch (hipSuccess when nothing to do).
hipError_t launch_gemv(const LaunchArgs &a);
hipError_t launch_gemm(const LaunchArgs &a);
hipError_t launch_fill_zero(void *Y, int64_t bytes, hipStream_t stream);

// Compute units of the current device (cached per device, thread-safe).
int num_cus();
// Workgroups of `kernel` (block `threads`, `lds` dynamic LDS bytes) that one
// compute unit holds at once; cached per (kernel, threads, lds, device).
int resident_blocks(const void *kernel, int threads, int lds);

}  // namespace lowbit
