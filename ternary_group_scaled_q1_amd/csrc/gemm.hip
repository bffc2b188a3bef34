// Prefill GEMM  Y[m][n] = sum_k X[m][k] t[n][k] s[n][k/128]  for large M.
//
// Prompt processing is compute-bound (aberweb.com page, summary section 3),
// so this path is a dense contraction on the matrix cores: the activation
// tile (128 tokens x 128 k, one weight group) is staged in LDS, each wave
// decodes its own weight operands straight from the packed bits in registers
// into exact +-1 / 0 f16/bf16 halves and issues v_mfma_f32_16x16x32.  The
// FP16 scale is applied once per group in fp32: each group accumulates into
// a fresh tile that is then added as s * tile (products exact, the scale is
// never rounded to bf16).
//
// Workgroup = 4 waves = 128 x 128 outputs; wave (wm, wn) owns 64 x 64 =
// 4 x 4 MFMA tiles, so every decoded weight operand feeds 4 MFMAs.  The 1-D
// block id is remapped so that each XCD walks a contiguous run of tiles that
// share activation rows (their L2 holds them).
//
// Ternary base-3 bytes (5 trits per byte) are decoded with a 243-entry LDS
// table giving the five (sign, non-zero) bit pairs of a byte at bits
// 15-2i / 14-2i; a shift by 2i and a mask then give the operand half 2t of
// trit i.  In a full 640-trit segment byte b carries trit i of group i at
// offset b, so one table lookup serves five groups.
#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

constexpr int kBM = 128, kBN = 128;
constexpr int kThreads = 256;
constexpr int kXStride = 136;  // halves per LDS activation row (128 + 8 pad)

struct GemmParams {
  const uint8_t *W;
  const uint8_t *Sc;  // plane B (may be only 2-byte aligned for tq5)
  const uint16_t *X;
  void *Y;
  int M, N, K, G;
  int tiles_m, tiles_n;
  int y_f16;
  // tq5 geometry
  int s_full, L_tail, b_tail, rowbytes;
};

__device__ __forceinline__ uint16_t load_scale(const GemmParams &p, int n, int g) {
  const uint8_t *b = p.Sc + ((int64_t)n * p.G + g) * 2;
  return uint16_t(b[0] | (uint16_t(b[1]) << 8));
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The activation tile of one group (128 rows x 128 k) as 16-byte cells: each
// thread holds 8 of the tile's 2048 cells in registers between the global
// load and the LDS store, so the next group's loads overlap this group's MFMAs.
struct XRegs {
  u4_t v[8];
};

__device__ __forceinline__ void x_load(const GemmParams &p, XRegs &r, int m0, int g) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    const int row = idx >> 4, c16 = idx & 15;
    const bool in = m0 + row < p.M && g < p.G;
    const u4_t *src = reinterpret_cast<const u4_t *>(p.X + (in ? (int64_t)(m0 + row) * p.K + 128 * g + 8 * c16 : 0));
    const u4_t v = *src;
    const u4_t z = {0u, 0u, 0u, 0u};
    r.v[i] = in ? v : z;
  }
}

// Store the cells; for q1 also minus the sum over k % 4 in {2, 3} of every row
// (16 consecutive lanes hold one row's 16 cells).
template <int FMT, bool BF>
__device__ __forceinline__ void x_store(const XRegs &r, uint16_t *xs, float *corr) {
#pragma unroll
  for (int i = 0; i < 8; ++i) {
    const int idx = threadIdx.x + i * kThreads;
    const int row = idx >> 4, c16 = idx & 15;
    *reinterpret_cast<u4_t *>(xs + row * kXStride + 8 * c16) = r.v[i];
    if constexpr (FMT == 1) {
      const u4_t v = r.v[i];
      float c = (x_to_float(uint16_t(v.y), BF) + x_to_float(uint16_t(v.y >> 16), BF)) +
                (x_to_float(uint16_t(v.w), BF) + x_to_float(uint16_t(v.w >> 16), BF));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) c += __shfl_xor(c, o, 16);
      if (c16 == 0) corr[row] = -c;
    }
  }
}

// 4 k-steps of MFMAs for one group from LDS tile xs into fresh tiles (q1:
// seeded with -corr of each row), then acc += s * tile.  Bop(u, nb) returns
// the B operand (16 weight rows x 32 k) of n-block nb for k-step u.
template <int FMT, bool BF, class Bop>
__device__ __forceinline__ void group_mma(const uint16_t *xs, const float *corr, const float (&sc)[4],
                                          f4_t (&acc)[4][4], Bop bop) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave >> 1;
  const int j = lane & 15, q = lane >> 4;
  f4_t cg[4][4];
  f4_t init[4];
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    if constexpr (FMT == 1) {
      const float4 c = *reinterpret_cast<const float4 *>(corr + wm * 64 + 16 * mb + 4 * q);
      init[mb] = f4_t{c.x, c.y, c.z, c.w};
    } else {
      init[mb] = f4_t{0.f, 0.f, 0.f, 0.f};
    }
  }
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u4_t A[4], B[4];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      A[mb] = *reinterpret_cast<const u4_t *>(xs + (wm * 64 + 16 * mb + j) * kXStride + 32 * u + 8 * q);
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) B[nb] = bop(u, nb);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < 4; ++nb) cg[mb][nb] = mfma16x16x32<BF>(A[mb], B[nb], u == 0 ? init[mb] : cg[mb][nb]);
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[mb][nb][e] = fmaf(sc[nb], cg[mb][nb][e], acc[mb][nb][e]);
}

// Weight words of one chunk (4 groups) for this lane's 4 n-blocks, and their scales.
template <int FMT>
struct WChunk {
  uint32_t w[4][FMT == 1 ? 4 : 8];
  uint32_t s[4][2];
};

template <int FMT>
__device__ __forceinline__ void w_load(const GemmParams &p, WChunk<FMT> &wc, const int (&tileT)[4],
                                       const int (&RT)[4], int c) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  constexpr int WPU = FMT == 1 ? 4 : 8;
  const int64_t unit = FMT == 1 ? 16 : 32;
  const int Gc = uni(min(4, p.G - 4 * c));
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int R = RT[nb];
    if (R == 0 || c >= (p.G + 3) / 4) {
#pragma unroll
      for (int i = 0; i < WPU; ++i) wc.w[nb][i] = 0;
      wc.s[nb][0] = wc.s[nb][1] = 0;
      continue;
    }
    const uint8_t *blk = p.W + 16 * (int64_t)tileT[nb] * p.G * unit + (int64_t)R * 4 * c * unit;
    if (R == 16 && Gc == 4 && (p.G & 3) == 0) {
      const u4_t v0 = *(reinterpret_cast<const u4_t *>(blk) + lane);
      wc.w[nb][0] = v0.x; wc.w[nb][1] = v0.y; wc.w[nb][2] = v0.z; wc.w[nb][3] = v0.w;
      if constexpr (FMT == 2) {
        const u4_t v1 = *(reinterpret_cast<const u4_t *>(blk + 1024) + lane);
        wc.w[nb][4] = v1.x; wc.w[nb][5] = v1.y; wc.w[nb][6] = v1.z; wc.w[nb][7] = v1.w;
      }
      const u2_t sv = *reinterpret_cast<const u2_t *>(p.Sc + ((int64_t)(16 * tileT[nb] + j) * p.G + 4 * c) * 2);
      wc.s[nb][0] = sv.x; wc.s[nb][1] = sv.y;
    } else {
      const bool row_ok = j < R;
      const int jj = min(j, R - 1);
      const uint32_t *base = reinterpret_cast<const uint32_t *>(blk);
      uint32_t h[4];
#pragma unroll
      for (int gg = 0; gg < 4; ++gg) {
        const int g2 = min(gg, Gc - 1);
        const bool ok = row_ok && gg < Gc;
        if constexpr (FMT == 1) {
          const uint32_t w = base[(q * R + jj) * Gc + g2];
          wc.w[nb][gg] = ok ? w : 0u;
        } else {
          const int hh = g2 >> 1, Gh = min(2, Gc - 2 * hh);
          const uint32_t *hb = base + R * 16 * hh + ((q * R + jj) * Gh + (g2 - 2 * hh)) * 2;
          const uint32_t w0 = hb[0], w1 = hb[1];
          wc.w[nb][2 * gg + 0] = ok ? w0 : 0u;
          wc.w[nb][2 * gg + 1] = ok ? w1 : 0u;
        }
        const uint32_t sv = load_scale(p, 16 * tileT[nb] + jj, 4 * c + g2);
        h[gg] = ok ? sv : 0u;
      }
      wc.s[nb][0] = h[0] | (h[1] << 16);
      wc.s[nb][1] = h[2] | (h[3] << 16);
    }
  }
}

template <int FMT, bool BF>
__global__ void __launch_bounds__(kThreads) gemm_kernel(GemmParams p) {
  __shared__ __align__(16) uint16_t xs[2][kBM * kXStride];
  __shared__ __align__(16) float corr[2][kBM];
  __shared__ uint16_t lut[256];

  const int tile = xcd_swizzle(blockIdx.x, gridDim.x);
  const int tm = tile / p.tiles_n, tn = tile - tm * p.tiles_n;
  const int m0 = tm * kBM, n0 = tn * kBN;
  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wn = wave & 1;
  const int j = lane & 15, q = lane >> 4;

  if constexpr (FMT == 3) {
    for (int v = threadIdx.x; v < 256; v += kThreads) {
      uint32_t f = 0;
      int d = v;
      for (int i = 0; i < 5; ++i) {
        const int di = d % 3;
        d /= 3;
        const uint32_t sign = di == 0, nz = di != 1;
        f |= (sign << (15 - 2 * i)) | (nz << (14 - 2 * i));
      }
      lut[v] = uint16_t(v < 243 ? f : 0);
    }
  }

  // Row tiles (16 rows) of this wave's 4 n-blocks (wave-uniform).
  int tileT[4], RT[4];
#pragma unroll
  for (int nb = 0; nb < 4; ++nb) {
    const int n = n0 + wn * 64 + 16 * nb;
    tileT[nb] = uni(n / 16);
    RT[nb] = uni(n < p.N ? min(16, p.N - n) : 0);
  }

  f4_t acc[4][4];
#pragma unroll
  for (int a = 0; a < 4; ++a)
#pragma unroll
    for (int b = 0; b < 4; ++b) acc[a][b] = f4_t{0.f, 0.f, 0.f, 0.f};

  XRegs xr;
  x_load(p, xr, m0, 0);
  x_store<FMT, BF>(xr, xs[0], corr[0]);
  __syncthreads();

  if constexpr (FMT == 1 || FMT == 2) {
    const int chunks = (p.G + 3) / 4;
    WChunk<FMT> wa, wb;
    w_load<FMT>(p, wa, tileT, RT, 0);
    for (int c = 0; c < chunks; ++c) {
      w_load<FMT>(p, wb, tileT, RT, c + 1);  // next chunk in flight
#pragma unroll
      for (int gi = 0; gi < 4; ++gi) {
        const int g = 4 * c + gi;
        if (g >= p.G) break;
        const int buf = g & 1;
        if (g + 1 < p.G) x_load(p, xr, m0, g + 1);
        float sc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) sc[nb] = half_to_float(uint16_t(wa.s[nb][gi >> 1] >> (16 * (gi & 1))));
        group_mma<FMT, BF>(xs[buf], corr[buf], sc, acc, [&](int u, int nb) -> u4_t {
          if constexpr (FMT == 1) return q1_operand<BF>(wa.w[nb][gi], u);
          else return tq2_operand(wa.w[nb][2 * gi + (u >> 1)], u);
        });
        if (g + 1 < p.G) x_store<FMT, BF>(xr, xs[buf ^ 1], corr[buf ^ 1]);
        __syncthreads();
      }
      wa = wb;
    }
  } else {
    for (int seg = 0; seg * 5 < p.G; ++seg) {
      const bool full = seg < p.s_full;
      uint32_t d5[4][16];
      if (full) {
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int R = RT[nb];
          const bool row_ok = j < R;
          const int jj = min(j, max(R - 1, 0));
          const uint8_t *sb = p.W + 16 * (int64_t)tileT[nb] * p.rowbytes + (int64_t)R * 128 * seg;
          u4_t v0 = {0u, 0u, 0u, 0u}, v1 = {0u, 0u, 0u, 0u};
          if (R > 0) {
            v0 = *reinterpret_cast<const u4_t *>(sb + (q * R + jj) * 16);
            v1 = *reinterpret_cast<const u4_t *>(sb + R * 64 + (q * R + jj) * 16);
          }
          const uint32_t wds[8] = {row_ok ? v0.x : 0u, row_ok ? v0.y : 0u, row_ok ? v0.z : 0u, row_ok ? v0.w : 0u,
                                   row_ok ? v1.x : 0u, row_ok ? v1.y : 0u, row_ok ? v1.z : 0u, row_ok ? v1.w : 0u};
#pragma unroll
          for (int u = 0; u < 4; ++u)
#pragma unroll
            for (int pr = 0; pr < 4; ++pr) {
              const int w0 = 8 * u + 2 * pr;  // lane byte of weight e = 2pr of step u
              const uint32_t b0 = (wds[w0 >> 2] >> (8 * (w0 & 3))) & 0xFF;
              const uint32_t b1 = (wds[(w0 + 1) >> 2] >> (8 * ((w0 + 1) & 3))) & 0xFF;
              d5[nb][u * 4 + pr] = uint32_t(lut[b0]) | (uint32_t(lut[b1]) << 16);
            }
        }
      }
      for (int gs = 0; gs < 5; ++gs) {
        const int g = 5 * seg + gs;
        if (g >= p.G) break;
        const int buf = g & 1;
        if (g + 1 < p.G) x_load(p, xr, m0, g + 1);
        float sc[4];
#pragma unroll
        for (int nb = 0; nb < 4; ++nb) {
          const int n = 16 * tileT[nb] + min(j, max(RT[nb] - 1, 0));
          const float sv = RT[nb] > 0 ? half_to_float(load_scale(p, n, g)) : 0.f;
          sc[nb] = j < RT[nb] ? sv : 0.f;
        }
        if (full) {
          group_mma<FMT, BF>(xs[buf], corr[buf], sc, acc, [&](int u, int nb) -> u4_t {
            u4_t b;
            b.x = tq5_pair(d5[nb][u * 4 + 0], gs);
            b.y = tq5_pair(d5[nb][u * 4 + 1], gs);
            b.z = tq5_pair(d5[nb][u * 4 + 2], gs);
            b.w = tq5_pair(d5[nb][u * 4 + 3], gs);
            return b;
          });
        } else {
          // Tail segment, row-major bytes: offset kt -> byte kt % B, digit kt / B.
          group_mma<FMT, BF>(xs[buf], corr[buf], sc, acc, [&](int u, int nb) -> u4_t {
            uint32_t h[8];
            const int R = RT[nb];
            const int jj = min(j, max(R - 1, 0));
            const uint8_t *tb =
                p.W + 16 * (int64_t)tileT[nb] * p.rowbytes + (int64_t)R * 128 * p.s_full + (int64_t)jj * p.b_tail;
#pragma unroll
            for (int e = 0; e < 8; ++e) {
              const int kt = 128 * (g - 5 * p.s_full) + 32 * u + 8 * q + e;
              const int b = kt % p.b_tail, dig = kt / p.b_tail;
              int v = R > 0 ? tb[b] : 121;
              for (int t = 0; t < dig; ++t) v /= 3;
              const int d = v % 3;
              h[e] = (j >= R || d == 1) ? 0u : (d == 2 ? 0x4000u : 0xC000u);
            }
            u4_t b;
            b.x = h[0] | (h[1] << 16);
            b.y = h[2] | (h[3] << 16);
            b.z = h[4] | (h[5] << 16);
            b.w = h[6] | (h[7] << 16);
            return b;
          });
        }
        if (g + 1 < p.G) x_store<FMT, BF>(xr, xs[buf ^ 1], corr[buf ^ 1]);
        __syncthreads();
      }
    }
  }

  const float mul = FMT == 1 ? 1.f : 0.5f;  // ternary operands carry 2t
  const int wm = wave >> 1;
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < 4; ++nb) {
      const int n = n0 + wn * 64 + 16 * nb + j;
      if (n >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = m0 + wm * 64 + 16 * mb + 4 * q + e;
        if (m >= p.M) continue;
        const float v = acc[mb][nb][e] * mul;
        if (p.y_f16) reinterpret_cast<uint16_t *>(p.Y)[(int64_t)m * p.N + n] = float_to_half_rne(v);
        else reinterpret_cast<float *>(p.Y)[(int64_t)m * p.N + n] = v;
      }
    }
}

template <int FMT, bool BF>
hipError_t launch_t(const LaunchArgs &a) {
  GemmParams p{};
  p.W = a.W;
  p.Sc = a.W + plane_a_bytes(a.fmt, a.N, a.K);
  p.X = a.X;
  p.Y = a.Y;
  p.M = int(a.M); p.N = int(a.N); p.K = int(a.K); p.G = int(a.K / kGroup);
  p.tiles_m = int((a.M + kBM - 1) / kBM);
  p.tiles_n = int((a.N + kBN - 1) / kBN);
  p.y_f16 = a.y_f16;
  const Tq5Geom t = tq5_geom(a.K);
  p.s_full = int(t.s_full); p.L_tail = int(t.L_tail); p.b_tail = int(t.b_tail); p.rowbytes = int(t.rowbytes);
  const int grid = p.tiles_m * p.tiles_n;
  hipLaunchKernelGGL((gemm_kernel<FMT, BF>), dim3(grid), dim3(kThreads), 0, a.stream, p);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemm(const LaunchArgs &a) {
  switch (a.fmt * 2 + (a.x_bf16 ? 1 : 0)) {
    case 2: return launch_t<1, false>(a);
    case 3: return launch_t<1, true>(a);
    case 4: return launch_t<2, false>(a);
    case 5: return launch_t<2, true>(a);
    case 6: return launch_t<3, false>(a);
    case 7: return launch_t<3, true>(a);
  }
  return hipErrorInvalidValue;
}

namespace {
__global__ void fill_zero_kernel(uint32_t *p, int64_t words) {
  for (int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x; i < words; i += (int64_t)gridDim.x * blockDim.x)
    p[i] = 0;
}
__global__ void fill_zero_bytes_kernel(uint8_t *p, int64_t bytes) {
  const int64_t i = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (i < bytes) p[i] = 0;
}
}  // namespace

hipError_t launch_fill_zero(void *Y, int64_t bytes, hipStream_t stream) {
  if (bytes <= 0) return hipSuccess;
  const uintptr_t addr = reinterpret_cast<uintptr_t>(Y);
  if ((addr & 3) == 0 && (bytes & 3) == 0) {
    const int64_t words = bytes / 4;
    const int grid = int(words / 256 + 1 < 4096 ? words / 256 + 1 : 4096);
    hipLaunchKernelGGL(fill_zero_kernel, dim3(grid), dim3(256), 0, stream, static_cast<uint32_t *>(Y), words);
  } else {
    hipLaunchKernelGGL(fill_zero_bytes_kernel, dim3(int((bytes + 255) / 256)), dim3(256), 0, stream,
                       static_cast<uint8_t *>(Y), bytes);
  }
  return hipGetLastError();
}

}  // namespace lowbit
