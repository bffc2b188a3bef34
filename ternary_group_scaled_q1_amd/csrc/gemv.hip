// Decode GEMV  Y[m][n] = sum_k X[m][k] t[n][k] s[n][k/128]  for M <= 16 tokens.
//
// The decode step is bound by streaming the packed weights from HBM (the
// pages: memory bandwidth, not compute, limits token generation; aberweb.com
// page, section 2 and summary section 3).  The kernel therefore reads every
// weight byte exactly once with 16-byte-per-lane coalesced loads (one 1 KB
// wave load per chunk of 4 groups x 16 rows), decodes the bits in registers
// with one shift and one bitwise op per pair of weights (device.hpp), and
// lets the matrix cores do the multiply-adds: a v_mfma_f32_16x16x32 takes 16
// weight rows x 32 k as its B operand and up to 16 tokens x 32 k of x as its
// A operand.  The sign decode happens inside the kernel; no dense weight
// tensor exists anywhere (aberweb.com page, section 4.1).
//
// Per group of 128 weights the 4 k-steps accumulate into a fresh fp32 tile,
// which is then scaled by the group's FP16 scale in fp32 and added to the
// running sum (products exact, one fp32 rounding per group).
//
// Work split: a workgroup of 8 waves stages x (up to 16 tokens) in LDS as
// [k/8][token][8] 16-byte cells.  Waves form P = 8/S wave-rows of S waves;
// a wave-row owns R row tiles (16R rows) at a time and its S waves split the
// K chunks, reducing their partial sums through LDS in a fixed order
// (deterministic).  With S = 1 and x resident in LDS every wave runs its own
// persistent loop over row tiles.
#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

struct GemvParams {
  const uint8_t *W;    // plane A
  const uint16_t *Sc;  // plane B: FP16 scales [N][G]
  const uint16_t *X;   // [M][K]
  void *Y;             // [M][N]
  int M, N, K, G;
  int tiles, chunks;
  int S;               // waves splitting the chunks of a stage
  int SC;              // chunks staged in LDS at once (multiple of S)
  int n_stages;        // ceil(chunks / SC)
  int tilesets;        // ceil(tiles / R)
  int y_f16;
  // LDS byte offsets
  int off_corr, off_x, off_part, off_red;
};

struct LdsMap {
  int corr, x, part, red, total;
};

template <int FMT>
LdsMap lds_map(int M, int S, int SC, int R) {
  LdsMap m;
  int o = 16;  // zero cell
  m.corr = o;
  if (FMT == 1) o += SC * 4 * 16 * 4;
  m.x = o;
  o += M * SC * 1024;
  m.part = o;
  if (FMT == 1) o += SC * 64 * M * 4;
  o = (o + 15) & ~15;
  m.red = o;
  if (S > 1) o += kWaves * R * 4 * 64 * 4;
  m.total = o;
  return m;
}

// Stage chunks [c0, c0+nc) of x into LDS: cell (oct, m) = x[m][8*(32*c0 + oct) ..] at
// ((oct * M) + m) * 16.  For q1 also the per-(group, token) correction
//   corr[gs][m] = sum of x[m][k] over the group's k with k % 4 in {2, 3}
// (the weights the q1 operand feeds as t + 1 instead of t).
template <int FMT, bool BF>
__device__ void stage_x(const GemvParams &p, char *lds, int c0, int nc) {
  const int M = p.M;
  const int oct_total = nc * 64;
  const int k0 = c0 * 512;
  uint4 *xl = reinterpret_cast<uint4 *>(lds + p.off_x);
  float *part = reinterpret_cast<float *>(lds + p.off_part);
  for (int idx = threadIdx.x; idx < oct_total * M; idx += kThreads) {
    const int oct = idx / M, m = idx - oct * M;
    const int k = k0 + oct * 8;
    uint4 v = make_uint4(0, 0, 0, 0);
    if (k < p.K) v = *reinterpret_cast<const uint4 *>(p.X + (int64_t)m * p.K + k);
    xl[oct * M + m] = v;
    if constexpr (FMT == 1) {
      const float a = x_to_float(uint16_t(v.y), BF) + x_to_float(uint16_t(v.y >> 16), BF);
      const float b = x_to_float(uint16_t(v.w), BF) + x_to_float(uint16_t(v.w >> 16), BF);
      part[oct * M + m] = a + b;
    }
  }
  if constexpr (FMT == 1) {
    __syncthreads();
    float *corr = reinterpret_cast<float *>(lds + p.off_corr);
    for (int idx = threadIdx.x; idx < nc * 4 * 16; idx += kThreads) {
      const int gs = idx >> 4, m = idx & 15;
      float c = 0.f;
      if (m < M)
        for (int o = 0; o < 16; ++o) c += part[(gs * 16 + o) * M + m];
      corr[idx] = c;
    }
  }
}

// One wave: R row tiles starting at tile t0, chunk c (c_local inside the stage).
template <int FMT, bool BF, int MT, int R>
__device__ __forceinline__ void wave_chunk(const GemvParams &p, const char *lds, int t0, int c,
                                           int c_local, float (&yacc)[R][4]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const int Gc = min(4, p.G - 4 * c);
  constexpr int WPG = FMT == 1 ? 1 : 2;  // lane words per group
  uint32_t wb[R][4 * WPG];
  uint16_t sc[R][4];
  bool tile_ok[R];

  const int64_t unit = FMT == 1 ? 16 : 32;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = t0 + r;
    tile_ok[r] = t < p.tiles;
#pragma unroll
    for (int i = 0; i < 4 * WPG; ++i) wb[r][i] = 0;
#pragma unroll
    for (int i = 0; i < 4; ++i) sc[r][i] = 0;
    if (!tile_ok[r]) continue;
    const int RT = min(16, p.N - 16 * t);
    const int64_t blk = 16 * (int64_t)t * p.G * unit + (int64_t)RT * 4 * c * unit;
    const int n = 16 * t + j;
    if (RT == 16 && Gc == 4) {
      if constexpr (FMT == 1) {
        const uint4 v = *reinterpret_cast<const uint4 *>(p.W + blk + 16 * lane);
        wb[r][0] = v.x; wb[r][1] = v.y; wb[r][2] = v.z; wb[r][3] = v.w;
      } else {
        const uint4 v0 = *reinterpret_cast<const uint4 *>(p.W + blk + 16 * lane);
        const uint4 v1 = *reinterpret_cast<const uint4 *>(p.W + blk + 16 * 64 + 16 * lane);
        wb[r][0] = v0.x; wb[r][1] = v0.y; wb[r][2] = v0.z; wb[r][3] = v0.w;
        wb[r][4] = v1.x; wb[r][5] = v1.y; wb[r][6] = v1.z; wb[r][7] = v1.w;
      }
    } else if (j < RT) {
      const uint32_t *base = reinterpret_cast<const uint32_t *>(p.W + blk);
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        if (g >= Gc) break;
        if constexpr (FMT == 1) {
          wb[r][g] = base[(q * RT + j) * Gc + g];
        } else {
          const int hh = g >> 1, Gh = min(2, Gc - 2 * hh);
          const uint32_t *hb = base + RT * 16 * hh;
          wb[r][2 * g + 0] = hb[((q * RT + j) * Gh + (g - 2 * hh)) * 2 + 0];
          wb[r][2 * g + 1] = hb[((q * RT + j) * Gh + (g - 2 * hh)) * 2 + 1];
        }
      }
    }
    if (j < RT) {
      const uint16_t *srow = p.Sc + (int64_t)n * p.G + 4 * c;
      if (Gc == 4 && (p.G & 3) == 0) {
        const uint2 v = *reinterpret_cast<const uint2 *>(srow);
        sc[r][0] = uint16_t(v.x); sc[r][1] = uint16_t(v.x >> 16);
        sc[r][2] = uint16_t(v.y); sc[r][3] = uint16_t(v.y >> 16);
      } else {
#pragma unroll
        for (int g = 0; g < 4; ++g)
          if (g < Gc) sc[r][g] = srow[g];
      }
    }
  }

  // A-operand (x) addressing: lane (q, i) reads token i, k-octet 4u+q of group g.
  const int i = j;
  const bool xact = i < p.M;
  const int lane_x = p.off_x + (q * p.M + i) * 16;
  const float *corr = reinterpret_cast<const float *>(lds + p.off_corr);

#pragma unroll
  for (int g = 0; g < 4; ++g) {
    if (g >= Gc) break;
    f4_t acc[R];
#pragma unroll
    for (int u = 0; u < 4; ++u) {
      const int step = ((c_local * 4 + g) * 16 + 4 * u) * p.M * 16;
      const int addr = xact ? lane_x + step : 0;
      const u4_t a = *reinterpret_cast<const u4_t *>(lds + addr);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        if (!tile_ok[r]) continue;
        u4_t b;
        if constexpr (FMT == 1) b = q1_operand<BF>(wb[r][g], u);
        else b = tq2_operand(wb[r][2 * g + (u >> 1)], u);
        acc[r] = u == 0 ? mfma16x16x32_zero<BF>(a, b) : mfma16x16x32<BF>(a, b, acc[r]);
      }
    }
    float cr[4] = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == 1) {
      const float4 cv = *reinterpret_cast<const float4 *>(corr + (c_local * 4 + g) * 16 + 4 * q);
      cr[0] = cv.x; cr[1] = cv.y; cr[2] = cv.z; cr[3] = cv.w;
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if (!tile_ok[r]) continue;
      const float s = half_to_float(sc[r][g]);
#pragma unroll
      for (int e = 0; e < (MT == 1 ? 1 : 4); ++e) yacc[r][e] = fmaf(s, acc[r][e] - cr[e], yacc[r][e]);
    }
  }
}

template <int FMT, int MT, int R>
__device__ __forceinline__ void store_tileset(const GemvParams &p, int t0, const float (&yacc)[R][4]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const float mul = FMT == 1 ? 1.f : 0.5f;  // ternary operands carry 2t
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = 16 * (t0 + r) + j;
    if (t0 + r >= p.tiles || n >= p.N) continue;
#pragma unroll
    for (int e = 0; e < (MT == 1 ? 1 : 4); ++e) {
      const int m = 4 * q + e;
      if (m >= p.M) continue;
      const float v = yacc[r][e] * mul;
      if (p.y_f16) reinterpret_cast<uint16_t *>(p.Y)[(int64_t)m * p.N + n] = float_to_half_rne(v);
      else reinterpret_cast<float *>(p.Y)[(int64_t)m * p.N + n] = v;
    }
  }
}

template <int FMT, bool BF, int MT, int R>
__global__ void __launch_bounds__(kThreads) gemv_kernel(GemvParams p) {
  extern __shared__ __align__(16) char lds[];
  const int wave = threadIdx.x >> 6;
  const int lane = threadIdx.x & 63;
  if (threadIdx.x < 4) reinterpret_cast<uint32_t *>(lds)[threadIdx.x] = 0;  // zero cell

  const int S = p.S, P = kWaves / S;
  const int pr = wave / S, s = wave - pr * S;

  if (S == 1 && p.n_stages == 1) {
    // x resident; every wave runs its own loop over tile sets.
    stage_x<FMT, BF>(p, lds, 0, p.chunks);
    __syncthreads();
    for (int ts = blockIdx.x * kWaves + wave; ts < p.tilesets; ts += gridDim.x * kWaves) {
      float yacc[R][4] = {};
      for (int c = 0; c < p.chunks; ++c) wave_chunk<FMT, BF, MT, R>(p, lds, ts * R, c, c, yacc);
      store_tileset<FMT, MT, R>(p, ts * R, yacc);
    }
    return;
  }

  const int rowblocks = (p.tilesets + P - 1) / P;
  bool staged_once = false;
  for (int rb = blockIdx.x; rb < rowblocks; rb += gridDim.x) {
    const int ts = rb * P + pr;
    const bool ts_ok = ts < p.tilesets;
    float yacc[R][4] = {};
    for (int st = 0; st < p.n_stages; ++st) {
      const int c0 = st * p.SC;
      const int nc = min(p.SC, p.chunks - c0);
      if (p.n_stages > 1 || !staged_once) {
        __syncthreads();
        stage_x<FMT, BF>(p, lds, c0, nc);
        __syncthreads();
        staged_once = true;
      }
      if (ts_ok)
        for (int cl = s; cl < nc; cl += S) wave_chunk<FMT, BF, MT, R>(p, lds, ts * R, c0 + cl, cl, yacc);
    }
    if (S == 1) {
      if (ts_ok) store_tileset<FMT, MT, R>(p, ts * R, yacc);
    } else {
      float *red = reinterpret_cast<float *>(lds + p.off_red);
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) red[((wave * R + r) * 4 + e) * 64 + lane] = yacc[r][e];
      __syncthreads();
      if (s == 0 && ts_ok) {
        float tot[R][4];
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) {
            float v = 0.f;
            for (int s2 = 0; s2 < S; ++s2) v += red[(((pr * S + s2) * R + r) * 4 + e) * 64 + lane];
            tot[r][e] = v;
          }
        store_tileset<FMT, MT, R>(p, ts * R, tot);
      }
      __syncthreads();
    }
  }
}

template <int FMT, bool BF, int MT, int R>
hipError_t launch_t(const LaunchArgs &a) {
  GemvParams p{};
  const int64_t G = a.K / kGroup;
  p.W = a.W;
  p.Sc = reinterpret_cast<const uint16_t *>(a.W + plane_a_bytes(a.fmt, a.N, a.K));
  p.X = a.X;
  p.Y = a.Y;
  p.M = int(a.M); p.N = int(a.N); p.K = int(a.K); p.G = int(G);
  p.tiles = int((a.N + 15) / 16);
  p.chunks = int((G + 3) / 4);
  p.tilesets = (p.tiles + R - 1) / R;
  p.y_f16 = a.y_f16;

  // K split: enough (tile set, split) pairs to fill 256 CUs x 8 waves.
  int S = 1;
  while (S < 8 && (int64_t)p.tilesets * S < 2048 && S * 2 <= p.chunks && MT * S * 2 <= 32) S *= 2;
  // Chunks staged per stage: all of them if the LDS map fits in 64 KB, else
  // the largest multiple of S that does.
  int SC = (p.chunks + S - 1) / S * S;
  while (SC > S && lds_map<FMT>(p.M, S, SC, R).total > 64 * 1024) SC -= S;
  p.S = S;
  p.SC = SC;
  p.n_stages = (p.chunks + SC - 1) / SC;
  const LdsMap m = lds_map<FMT>(p.M, S, SC, R);
  p.off_corr = m.corr; p.off_x = m.x; p.off_part = m.part; p.off_red = m.red;

  const int P = kWaves / S;
  int grid;
  if (S == 1 && p.n_stages == 1) grid = (p.tilesets + kWaves - 1) / kWaves;
  else grid = (p.tilesets + P - 1) / P;
  const int per_cu = m.total <= 40 * 1024 ? 3 : (m.total <= 64 * 1024 ? 2 : 1);
  grid = max(1, min(grid, 256 * per_cu));
  hipLaunchKernelGGL((gemv_kernel<FMT, BF, MT, R>), dim3(grid), dim3(kThreads), m.total, a.stream, p);
  return hipGetLastError();
}

template <int FMT, bool BF>
hipError_t launch_mt(const LaunchArgs &a) {
  if (a.M <= 1) return launch_t<FMT, BF, 1, 2>(a);
  if (a.M <= 4) return launch_t<FMT, BF, 4, 2>(a);
  return launch_t<FMT, BF, 16, 2>(a);
}

}  // namespace

hipError_t launch_gemv(const LaunchArgs &a) {
  // Token blocks of at most 16 rows share one pass over the weights.
  for (int64_t m0 = 0; m0 < a.M; m0 += 16) {
    LaunchArgs b = a;
    b.M = a.M - m0 < 16 ? a.M - m0 : 16;
    b.X = a.X + m0 * a.K;
    b.Y = static_cast<char *>(a.Y) + m0 * a.N * (a.y_f16 ? 2 : 4);
    hipError_t e;
    if (a.fmt == 1) e = a.x_bf16 ? launch_mt<1, true>(b) : launch_mt<1, false>(b);
    else e = a.x_bf16 ? launch_mt<2, true>(b) : launch_mt<2, false>(b);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lowbit
