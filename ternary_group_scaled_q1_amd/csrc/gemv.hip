// Decode GEMV  Y[m][n] = sum_k X[m][k] t[n][k] s[n][k/128]  for M <= 16 tokens.
//
// Token generation is bound by streaming the packed weights from HBM
// (aberweb.com page, section 2 and summary section 3), so the kernel reads
// every weight byte exactly once, as 16-byte-per-lane coalesced loads (a
// full chunk of 4 groups x 16 rows is one contiguous 1 KB wave load),
// keeps the next unit's loads in flight while it works on the current one,
// decodes the bits in registers with one shift and one bitwise op per pair
// of weights (device.hpp), and lets the matrix cores do the multiply-adds:
// a v_mfma_f32_16x16x32 takes 16 weight rows x 32 k as its B operand and up
// to 16 tokens x 32 k of x as its A operand.  No dense weight tensor exists
// anywhere: the signs are decoded inside the kernel (aberweb.com page,
// section 4.1).
//
// Per group of 128 weights the 4 k-steps accumulate into a fresh fp32 tile
// that is scaled by the group's FP16 scale in fp32 and added to the running
// sum (exact products, one fp32 rounding per group).
//
// Work split: a workgroup of 8 waves stages x in LDS as [k/8][token][8]
// 16-byte cells, all of K at once when it fits (then the stage is loaded
// once per workgroup) or S chunks at a time.  The waves form P = 8/S
// wave-rows; a wave-row owns R row tiles (16R rows) at a time and its S
// waves split each stage's chunks, adding their partial sums through LDS in
// a fixed order, so results are deterministic.  All control flow that
// decides loads, MFMAs and barriers is wave-uniform.
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
  int S;         // waves splitting the chunks of a stage
  int SC;        // chunks per stage (multiple of S)
  int n_stages;  // ceil(chunks / SC)
  int tilesets;  // ceil(tiles / R)
  int y_f16;
  int off_corr, off_x, off_red;
};

struct LdsMap {
  int corr, x, red, total;
};

// x cells hold MTS token slots (MTS = 1, 4 or 16); lanes whose token slot is
// past MTS read a zero region as large as one chunk of cells.
inline LdsMap lds_map(int MTS, int S, int SC, int R, int E) {
  LdsMap m;
  int o = MTS == 16 ? 0 : 64 * 16 * MTS;
  m.corr = o;
  o += SC * 4 * 16 * 4;
  m.x = o;
  o += MTS * SC * 1024;
  m.red = o;
  if (S > 1) o += kWaves * R * E * 64 * 4;
  m.total = o;
  return m;
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Stage chunks [c0, c0 + nc) of x: cell (oct, m) holds x[m][k0 + 8 oct .. + 8] at
// byte off_x + (oct * MTS + m) * 16 (zeros past K and for m >= M).  One thread
// per (group, token slot) also sums the group's activations at k % 4 in {2, 3}:
// the q1 operand feeds those weights as t + 1, so minus that sum is stored in
// corr[group][token] and seeds the group's accumulator.
template <int FMT, bool BF, int MTS>
__device__ void stage_x(const GemvParams &p, char *lds, int c0, int nc) {
  const int k0 = c0 * 512;
  uint4 *xl = reinterpret_cast<uint4 *>(lds + p.off_x);
  float *corr = reinterpret_cast<float *>(lds + p.off_corr);
  // One thread per (token slot, k-octet); the 16 octets of a group sit in 16
  // consecutive lanes, which add up the group's correction by shuffles.
  const int cells = MTS * nc * 64;
  for (int base = 0; base < cells; base += kThreads) {
    const int idx = base + threadIdx.x;
    const int m = idx / (nc * 64), oct = idx - m * (nc * 64);
    const int k = k0 + oct * 8;
    const bool live = idx < cells;
    const bool in = live && k < p.K && m < p.M;
    const u4_t *src = reinterpret_cast<const u4_t *>(p.X + (in ? (int64_t)m * p.K + k : 0));
    u4_t v = *src;
    const u4_t z = {0u, 0u, 0u, 0u};
    v = in ? v : z;
    if (live) *reinterpret_cast<u4_t *>(xl + oct * MTS + m) = v;
    if constexpr (FMT == 1) {
      float c = (x_to_float(uint16_t(v.y), BF) + x_to_float(uint16_t(v.y >> 16), BF)) +
                (x_to_float(uint16_t(v.w), BF) + x_to_float(uint16_t(v.w >> 16), BF));
#pragma unroll
      for (int o = 1; o < 16; o <<= 1) c += __shfl_xor(c, o, 16);
      if (live && (oct & 15) == 0) corr[(oct >> 4) * 16 + m] = -c;
    }
  }
  if constexpr (FMT == 1) {
    // Token slots without a token get a zero correction.
    for (int idx = threadIdx.x; idx < nc * 4 * (16 - MTS); idx += kThreads) {
      const int gs = idx / (16 - MTS), m = MTS + idx % (16 - MTS);
      corr[gs * 16 + m] = 0.f;
    }
  }
}

// Packed words and scales of R row tiles x one chunk (4 groups), for one lane.
template <int FMT, int R>
struct Unit {
  static constexpr int WPU = FMT == 1 ? 4 : 8;
  uint32_t w[R][WPU];
  uint32_t s[R][2];  // 4 FP16 scales
};

// Loads are issued without per-lane branches (ragged tiles clamp their
// addresses and zero the values afterwards): a divergent branch around a
// load makes the compiler wait for every outstanding load at the join, which
// would drain the prefetch ring.
template <int FMT, int R>
__device__ __forceinline__ void load_unit(const GemvParams &p, Unit<FMT, R> &u, int t0, int c, bool valid) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  constexpr int WPU = Unit<FMT, R>::WPU;
  const int64_t unit = FMT == 1 ? 16 : 32;
  const int Gc = uni(min(4, p.G - 4 * c));
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = uni(t0 + r);
    if (!valid || t >= p.tiles) {  // wave-uniform
#pragma unroll
      for (int i = 0; i < WPU; ++i) u.w[r][i] = 0;
      u.s[r][0] = u.s[r][1] = 0;
      continue;
    }
    const int RT = uni(min(16, p.N - 16 * t));
    const uint8_t *blk = p.W + 16 * (int64_t)t * p.G * unit + (int64_t)RT * 4 * c * unit;
    if (RT == 16 && Gc == 4 && (p.G & 3) == 0) {  // wave-uniform fast path
      const u4_t v0 = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(blk) + lane);
      u.w[r][0] = v0.x; u.w[r][1] = v0.y; u.w[r][2] = v0.z; u.w[r][3] = v0.w;
      if constexpr (FMT == 2) {
        const u4_t v1 = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(blk + 1024) + lane);
        u.w[r][4] = v1.x; u.w[r][5] = v1.y; u.w[r][6] = v1.z; u.w[r][7] = v1.w;
      }
      const u2_t sv = *reinterpret_cast<const u2_t *>(p.Sc + (int64_t)(16 * t + j) * p.G + 4 * c);
      u.s[r][0] = sv.x; u.s[r][1] = sv.y;
    } else {
      const bool row_ok = j < RT;
      const int jj = min(j, RT - 1);
      const uint32_t *base = reinterpret_cast<const uint32_t *>(blk);
      const uint16_t *srow = p.Sc + (int64_t)(16 * t + jj) * p.G + 4 * c;
      uint32_t h[4];
#pragma unroll
      for (int g = 0; g < 4; ++g) {
        const int gg = min(g, Gc - 1);
        const bool ok = row_ok && g < Gc;
        if constexpr (FMT == 1) {
          const uint32_t w = base[(q * RT + jj) * Gc + gg];
          u.w[r][g] = ok ? w : 0u;
        } else {
          const int hh = gg >> 1, Gh = min(2, Gc - 2 * hh);
          const uint32_t *hb = base + RT * 16 * hh + ((q * RT + jj) * Gh + (gg - 2 * hh)) * 2;
          const uint32_t w0 = hb[0], w1 = hb[1];
          u.w[r][2 * g + 0] = ok ? w0 : 0u;
          u.w[r][2 * g + 1] = ok ? w1 : 0u;
        }
        const uint32_t sv = srow[gg];
        h[g] = ok ? sv : 0u;
      }
      u.s[r][0] = h[0] | (h[1] << 16);
      u.s[r][1] = h[2] | (h[3] << 16);
    }
  }
}

// x operand cells of step (g, uu) sit at a compile-time offset from the
// lane's chunk base, so the LDS reads need no address arithmetic.
template <int FMT, bool BF, int R, int E, int MTS>
__device__ __forceinline__ void compute_unit(const GemvParams &p, const char *lds, const Unit<FMT, R> &u, int c_local,
                                             int xbase, float (&yacc)[R][4]) {
  const int q = (threadIdx.x & 63) >> 4;
  const float *corr = reinterpret_cast<const float *>(lds + p.off_corr) + c_local * 64 + 4 * q;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    // q1: the group's accumulator starts at -(sum of x fed as t + 1).
    f4_t init = {0.f, 0.f, 0.f, 0.f};
    if constexpr (FMT == 1) {
      if constexpr (E == 1) {
        init[0] = corr[g * 16];
      } else {
        const float4 cv = *reinterpret_cast<const float4 *>(corr + g * 16);
        init = f4_t{cv.x, cv.y, cv.z, cv.w};
      }
    }
    f4_t acc[R];
#pragma unroll
    for (int uu = 0; uu < 4; ++uu) {
      const u4_t a = *reinterpret_cast<const u4_t *>(lds + xbase + (g * 16 + 4 * uu) * MTS * 16);
#pragma unroll
      for (int r = 0; r < R; ++r) {
        u4_t b;
        if constexpr (FMT == 1) b = q1_operand<BF>(u.w[r][g], uu);
        else b = tq2_operand(u.w[r][2 * g + (uu >> 1)], uu);
        if constexpr (FMT == 1) acc[r] = mfma16x16x32<BF>(a, b, uu == 0 ? init : acc[r]);
        else acc[r] = uu == 0 ? mfma16x16x32_zero<BF>(a, b) : mfma16x16x32<BF>(a, b, acc[r]);
      }
    }
#pragma unroll
    for (int r = 0; r < R; ++r) {
      const float s = half_to_float(uint16_t(u.s[r][g >> 1] >> (16 * (g & 1))));
#pragma unroll
      for (int e = 0; e < E; ++e) yacc[r][e] = fmaf(s, acc[r][e], yacc[r][e]);
    }
  }
}

template <int FMT, int R, int E>
__device__ __forceinline__ void store_tiles(const GemvParams &p, int t0, const float (&yacc)[R][4]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const float mul = FMT == 1 ? 1.f : 0.5f;  // ternary operands carry 2t
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int n = 16 * (t0 + r) + j;
    if (n >= p.N) continue;
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int m = 4 * q + e;
      if (m >= p.M) continue;
      const float v = yacc[r][e] * mul;
      if (p.y_f16) reinterpret_cast<uint16_t *>(p.Y)[(int64_t)m * p.N + n] = float_to_half_rne(v);
      else reinterpret_cast<float *>(p.Y)[(int64_t)m * p.N + n] = v;
    }
  }
}

// Position of a wave in its flat sequence of units: tile set iteration it,
// stage st, slot kl inside the stage.  Advanced incrementally (no divisions).
struct Cursor {
  int it, st, kl;
};

__device__ __forceinline__ void advance(Cursor &c, int U, int n_stages) {
  if (++c.kl == U) {
    c.kl = 0;
    if (++c.st == n_stages) {
      c.st = 0;
      ++c.it;
    }
  }
}

// Each wave walks a flat sequence of units (tile set, chunk) with a ring of
// D units in flight: the loads of unit i + D - 1 are issued before unit i is
// computed, across chunk, stage and tile-set boundaries.
template <int FMT, bool BF, int MT, int R, int D>
__global__ void __launch_bounds__(kThreads, 4) gemv_kernel(GemvParams p) {
  constexpr int E = MT == 1 ? 1 : 4;     // accumulator elements that can hold a token
  constexpr int MTS = MT;                // token slots per x cell
  extern __shared__ __align__(16) char lds[];
  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  if constexpr (MTS < 16) {
    for (int i = threadIdx.x; i < 64 * MTS; i += kThreads) reinterpret_cast<uint4 *>(lds)[i] = make_uint4(0, 0, 0, 0);
  }

  const int S = uni(p.S), P = kWaves / S;
  const int pr = uni(wave / S), s = uni(wave - pr * S);
  const int U = uni(p.SC / S);          // unit slots per wave per stage
  const int KT = uni(p.n_stages * U);   // unit slots per wave per tile set
  const bool restage = p.n_stages > 1;
  const bool lockstep = restage || S > 1;
  const int rows_total = gridDim.x * P;  // wave-rows in the grid
  // Tile set of iteration it: consecutive wave-rows of one workgroup are
  // gridDim.x apart, so extra tile sets spread over all CUs.
  const int my_row = pr * gridDim.x + blockIdx.x;
  const int iters = lockstep ? (p.tilesets + rows_total - 1) / rows_total
                             : (p.tilesets - my_row + rows_total - 1) / rows_total;
  const int total = uni(iters * KT);
  // Token slots past MTS read the zero region; slots in [M, MTS) hold zeros.
  const bool xact = j < MTS;

  auto tile0 = [&](const Cursor &c) { return (c.it * rows_total + my_row) * R; };
  auto chunk = [&](const Cursor &c) { return c.st * p.SC + s + c.kl * S; };
  auto is_valid = [&](const Cursor &c) {
    return c.it * rows_total + my_row < p.tilesets && chunk(c) < p.chunks;
  };

  // First D - 1 units' loads go out before x is staged.
  float yacc[R][4];
  Unit<FMT, R> ring[D];
  Cursor ld = {0, 0, 0};
#pragma unroll
  for (int d = 0; d < D - 1; ++d) {
    load_unit<FMT, R>(p, ring[d], uni(tile0(ld)), uni(chunk(ld)), d < total && is_valid(ld));
    advance(ld, U, p.n_stages);
  }
  if (!restage) {
    stage_x<FMT, BF, MTS>(p, lds, 0, p.chunks);
    __syncthreads();
  }

  Cursor cu = {0, 0, 0};
  for (int i0 = 0; i0 < total; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      if (i >= total) break;
      load_unit<FMT, R>(p, ring[(d + D - 1) % D], uni(tile0(ld)), uni(chunk(ld)), i + D - 1 < total && is_valid(ld));
      advance(ld, U, p.n_stages);

      const int t0 = uni(tile0(cu));
      const int k_first = cu.st == 0 && cu.kl == 0;
      const int k_last = cu.st == p.n_stages - 1 && cu.kl == U - 1;
      if (k_first) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) yacc[r][e] = 0.f;
      }
      if (restage && cu.kl == 0) {
        __syncthreads();
        const int c0 = cu.st * p.SC;
        stage_x<FMT, BF, MTS>(p, lds, c0, min(p.SC, p.chunks - c0));
        __syncthreads();
      }
      if (is_valid(cu)) {
        const int c_local = s + cu.kl * S;
        const int xbase = xact ? p.off_x + (c_local * 64 * MTS + q * MTS + j) * 16 : 0;
        compute_unit<FMT, BF, R, E, MTS>(p, lds, ring[d], c_local, xbase, yacc);
      }
      if (k_last) {
        const bool ts_ok = t0 < p.tiles;
        if (S == 1) {
          if (ts_ok) store_tiles<FMT, R, E>(p, t0, yacc);
        } else {
          float *red = reinterpret_cast<float *>(lds + p.off_red);
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) red[((wave * R + r) * E + e) * 64 + lane] = yacc[r][e];
          __syncthreads();
          if (s == 0 && ts_ok) {
            float tot[R][4];
#pragma unroll
            for (int r = 0; r < R; ++r)
#pragma unroll
              for (int e = 0; e < E; ++e) {
                float v = 0.f;
                for (int s2 = 0; s2 < S; ++s2) v += red[(((pr * S + s2) * R + r) * E + e) * 64 + lane];
                tot[r][e] = v;
              }
            store_tiles<FMT, R, E>(p, t0, tot);
          }
          __syncthreads();
        }
      }
      advance(cu, U, p.n_stages);
    }
  }
}

// Host-side choice of (R, S): the smallest per-wave work (the makespan:
// tile sets per wave-row x R x chunks per wave), then fewer barriers.
template <int FMT, bool BF, int MT, int R, int D>
double make_plan(const LaunchArgs &a, GemvParams &p, int &grid, int &lds_bytes) {
  constexpr int E = MT == 1 ? 1 : 4;
  p = GemvParams{};
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
  const int cus = num_cus();
  const void *kern = reinterpret_cast<const void *>(&gemv_kernel<FMT, BF, MT, R, D>);

  double best = 1e300;
  GemvParams bp = p;
  int bgrid = 1, blds = 0;
  for (int S = 1; S <= 8; S *= 2) {
    if (S > 1 && S > p.chunks) break;
    GemvParams q = p;
    // Stage all chunks when the LDS map fits in 64 KB, else stream stages of
    // as many chunks as fit in 32 KB of x.
    int SC = (p.chunks + S - 1) / S * S;
    if (lds_map(MT, S, SC, R, E).total > 64 * 1024) {
      if (MT * S * 1024 > 32 * 1024) continue;
      SC = S;
      while (SC + S <= p.chunks && MT * (SC + S) * 1024 <= 32 * 1024) SC += S;
    }
    q.S = S;
    q.SC = SC;
    q.n_stages = (p.chunks + SC - 1) / SC;
    const LdsMap m = lds_map(MT, S, SC, R, E);
    q.off_corr = m.corr; q.off_x = m.x; q.off_red = m.red;
    const int P = kWaves / S;
    const int per_cu = resident_blocks(kern, kThreads, m.total);
    const int g = max(1, min((q.tilesets + P - 1) / P, cus * per_cu));
    const int64_t rows = (int64_t)g * P;
    // Makespan in units of (tile, chunk) work per wave, with a small charge
    // for workgroup barriers (K split or streamed stages).
    const double units = double((q.tilesets + rows - 1) / rows) * R * ((p.chunks + S - 1) / S);
    const double cost = units * ((S > 1 || q.n_stages > 1) ? 1.05 : 1.0);
    if (cost < best) {
      best = cost;
      bp = q;
      bgrid = g;
      blds = m.total;
    }
  }
  p = bp;
  grid = bgrid;
  lds_bytes = blds;
  // R = 1 reads the x operand from LDS once per MFMA instead of once per two.
  return best * (R == 1 ? 1.1 : 1.0);
}

template <int FMT, bool BF, int MT>
hipError_t launch_mt(const LaunchArgs &a) {
  GemvParams p1, p2;
  int g1, g2, l1, l2;
  // Ring depth: three units in flight for q1 (1 KB per tile each), two for
  // tq2 (2 KB per tile each) so that four waves per SIMD fit in registers.
  constexpr int D = FMT == 1 ? 3 : 2;
  const double c1 = make_plan<FMT, BF, MT, 1, D>(a, p1, g1, l1);
  const double c2 = make_plan<FMT, BF, MT, 2, D>(a, p2, g2, l2);
  if (c1 < c2)
    hipLaunchKernelGGL((gemv_kernel<FMT, BF, MT, 1, D>), dim3(g1), dim3(kThreads), l1, a.stream, p1);
  else
    hipLaunchKernelGGL((gemv_kernel<FMT, BF, MT, 2, D>), dim3(g2), dim3(kThreads), l2, a.stream, p2);
  return hipGetLastError();
}

template <int FMT, bool BF>
hipError_t launch_fmt(const LaunchArgs &a) {
  if (a.M <= 1) return launch_mt<FMT, BF, 1>(a);
  if (a.M <= 4) return launch_mt<FMT, BF, 4>(a);
  return launch_mt<FMT, BF, 16>(a);
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
    if (a.fmt == 1) e = a.x_bf16 ? launch_fmt<1, true>(b) : launch_fmt<1, false>(b);
    else e = a.x_bf16 ? launch_fmt<2, true>(b) : launch_fmt<2, false>(b);
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace lowbit
