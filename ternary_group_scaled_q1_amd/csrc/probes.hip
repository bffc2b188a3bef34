// Platform probes for the benchmark (measurement only; the product path never
// calls them): what one MI355X sustains with plain kernels, as context for
// the rooflines of the library's kernels.
//  * probe_stream_read: every lane streams 16-byte nontemporal loads over a
//    buffer, four in flight, and folds them into a value that is stored only
//    if it equals an impossible pattern (so the loads cannot be dropped).
//  * probe_mfma_bf16: every wave runs four independent chains of
//    v_mfma_f32_16x16x32_bf16; the B operand is a +-1 pattern that changes
//    every step (as decoded low-bit weights do), the A operand random bf16.
//  * probe_empty: a kernel that does nothing, for the launch cost.
//  * probe_tile_read: the decode kernels' weight stream without the
//    arithmetic: wave t reads tile t (tile_bytes, a multiple of 1 KB) 1 KB
//    per step with D steps in flight; mode 1 starts wave t at chunk t mod
//    (chunks per tile); mode 2 reads a chunk-major layout in which chunk c
//    of tile t sits at (c T + t) KB, so one step of all waves is contiguous.
// Built into libprobes.so, a library of its own next to liblowbit.so.
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace {

typedef uint32_t u4v __attribute__((ext_vector_type(4)));
typedef __bf16 b8v __attribute__((ext_vector_type(8)));
typedef float f4v __attribute__((ext_vector_type(4)));

__global__ void __launch_bounds__(512) stream_read_kernel(const u4v *p, int64_t n16, uint32_t *sink) {
  const int64_t stride = int64_t(gridDim.x) * blockDim.x;
  int64_t i = int64_t(blockIdx.x) * blockDim.x + threadIdx.x;
  uint32_t acc = 0;
  for (; i + 3 * stride < n16; i += 4 * stride) {
    const u4v a = __builtin_nontemporal_load(p + i);
    const u4v b = __builtin_nontemporal_load(p + i + stride);
    const u4v c = __builtin_nontemporal_load(p + i + 2 * stride);
    const u4v d = __builtin_nontemporal_load(p + i + 3 * stride);
    acc ^= a.x ^ a.y ^ a.z ^ a.w ^ b.x ^ b.y ^ b.z ^ b.w ^ c.x ^ c.y ^ c.z ^ c.w ^ d.x ^ d.y ^ d.z ^ d.w;
  }
  for (; i < n16; i += stride) {
    const u4v a = __builtin_nontemporal_load(p + i);
    acc ^= a.x ^ a.y ^ a.z ^ a.w;
  }
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

__global__ void __launch_bounds__(512) mfma_kernel(float *out, int iters) {
  const uint32_t lane = threadIdx.x & 63, seed = (blockIdx.x * 512u + threadIdx.x) * 2654435761u;
  u4v a;
  a.x = (seed ^ 0x3F803F80u) & 0xBFFFBFFFu;  // random bf16 with exponents near 1
  a.y = ((seed * 3u) ^ 0x3F003F00u) & 0xBFFFBFFFu;
  a.z = ((seed * 5u) ^ 0x3E803E80u) & 0xBFFFBFFFu;
  a.w = ((seed * 7u) ^ 0x3F403F40u) & 0xBFFFBFFFu;
  uint32_t w = seed ^ (lane * 0x01010101u);
  f4v c0 = {0.f, 0.f, 0.f, 0.f}, c1 = c0, c2 = c0, c3 = c0;
  for (int it = 0; it < iters; ++it) {
    u4v b;  // +-1 bf16 pairs from the sign bits of a rotating word
    b.x = (w & 0x80008000u) ^ 0xBF80BF80u;
    b.y = ((w << 1) & 0x80008000u) ^ 0xBF80BF80u;
    b.z = ((w << 2) & 0x80008000u) ^ 0xBF80BF80u;
    b.w = ((w << 3) & 0x80008000u) ^ 0xBF80BF80u;
    w = (w << 4) | (w >> 28);
    const b8v A = __builtin_bit_cast(b8v, a), B = __builtin_bit_cast(b8v, b);
    c0 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c0, 0, 0, 0);
    c1 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(B, A, c1, 0, 0, 0);
    c2 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(A, B, c2, 0, 0, 0);
    c3 = __builtin_amdgcn_mfma_f32_16x16x32_bf16(B, A, c3, 0, 0, 0);
  }
  const float s = c0[0] + c1[1] + c2[2] + c3[3];
  if (s == 1234.5f) out[blockIdx.x] = s;
}

__global__ void empty_kernel() {}

template <int D>
__global__ void __launch_bounds__(512) tile_read_kernel(const char *base, int64_t tile_bytes, int T, int mode,
                                                        uint32_t *sink) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int t = blockIdx.x * 8 + wave;
  if (t >= T) return;
  const int nch = int(tile_bytes >> 10);
  const int rot = mode == 1 ? t % nch : 0;
  auto at = [&](int c) {
    int cc = c + rot;
    if (cc >= nch) cc -= nch;
    const int64_t off = mode == 2 ? (int64_t(cc) * T + t) * 1024 : int64_t(t) * tile_bytes + int64_t(cc) * 1024;
    return reinterpret_cast<const u4v *>(base + off) + lane;
  };
  uint32_t acc = 0;
  u4v r[D];
#pragma unroll
  for (int d = 0; d < D; ++d) r[d] = __builtin_nontemporal_load(at(min(d, nch - 1)));
  for (int c0 = 0; c0 < nch; c0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      acc ^= r[d].x ^ r[d].y ^ r[d].z ^ r[d].w;
      r[d] = __builtin_nontemporal_load(at(min(c0 + d + D, nch - 1)));
    }
  }
#pragma unroll
  for (int d = 0; d < D; ++d) acc ^= r[d].x;
  if (acc == 0x9E3779B9u) sink[threadIdx.x] = acc;
}

}  // namespace

extern "C" {

// Reads `bytes` (a multiple of 16) from device memory `buf` with `grid`
// workgroups of 512 lanes on `stream`; sink: 2 KiB of device memory.
int probe_stream_read(const void *buf, int64_t bytes, void *sink, int grid, void *stream) {
  hipLaunchKernelGGL(stream_read_kernel, dim3(grid), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<const u4v *>(buf), bytes / 16, static_cast<uint32_t *>(sink));
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

// `grid` workgroups of 8 waves, each wave 4 x iters MFMAs of 16x16x32
// (16384 flops each); out: grid floats of device memory.
int probe_mfma_bf16(void *out, int iters, int grid, void *stream) {
  hipLaunchKernelGGL(mfma_kernel, dim3(grid), dim3(512), 0, static_cast<hipStream_t>(stream),
                     static_cast<float *>(out), iters);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

// Reads tiles * tile_bytes of device memory at buf (tile_bytes a positive
// multiple of 1024; depth 2 or 4; mode 0, 1 or 2 as above) with 8 waves per
// workgroup; sink: 2 KiB of device memory.  -2 for arguments out of range.
int probe_tile_read(const void *buf, int64_t tile_bytes, int tiles, int depth, int mode, void *sink, void *stream) {
  if (tile_bytes < 1024 || tile_bytes % 1024 || tiles < 1 || (depth != 2 && depth != 4) || mode < 0 || mode > 2)
    return -2;
  const dim3 grid((tiles + 7) / 8), block(512);
  const hipStream_t st = static_cast<hipStream_t>(stream);
  const char *b = static_cast<const char *>(buf);
  uint32_t *sk = static_cast<uint32_t *>(sink);
  if (depth == 2) hipLaunchKernelGGL(tile_read_kernel<2>, grid, block, 0, st, b, tile_bytes, tiles, mode, sk);
  else hipLaunchKernelGGL(tile_read_kernel<4>, grid, block, 0, st, b, tile_bytes, tiles, mode, sk);
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

int probe_empty(void *stream) {
  hipLaunchKernelGGL(empty_kernel, dim3(1), dim3(64), 0, static_cast<hipStream_t>(stream));
  return hipGetLastError() == hipSuccess ? 0 : -8;
}

}  // extern "C"
