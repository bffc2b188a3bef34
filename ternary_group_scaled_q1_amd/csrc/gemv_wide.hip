// Decode GEMV for 9..16 tokens: Y[m][n] = sum_k X[m][k] t[n][k] s[n][k/128].
//
// With 16 tokens the activations of one K range are as large as the weights
// that use them (16 x 5120 bf16 = 160 KB), too large to stage in LDS once per
// workgroup.  Here every wave loads the A operand of each MFMA straight from
// memory into registers: lane 16q + j reads the 16 bytes x[j][k0 + 8q .. +8]
// of the k-step, which the L2 (and the CU's L1 when neighbouring waves walk
// the same groups) serves to all waves that share the K range.  No LDS
// staging and no barriers, except one at the end when waves that split K add
// their partial sums.
//
// Unit of work: R row tiles (16 rows each) x one group of 128 weights.  Per
// unit a lane holds its tiles' packed words of that group (q1: 4 bytes, tq2:
// 8 bytes per tile), their FP16 scales and 4 x 16 bytes of x; a ring of D
// units keeps the loads of the next units in flight while one is computed.
// The weights decode to exact +-1 (q1) or 2t (tq2) f16/bf16 operands with one
// shift and one bitwise op per pair (device.hpp), four k-steps of
// v_mfma_f32_16x16x32 fill a fresh fp32 tile per (tile, group), and the
// group's FP16 scale is applied to it in fp32 (exact products, one rounding
// per group), as on the aberweb.com page, section 4.1: the signs are decoded
// inside the kernel and no dense weight tensor exists.
#include "device.hpp"
#include "gemv_common.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

struct WideParams {
  MatSet ms;           // the matrices (row tiles numbered across them)
  const uint16_t *X;   // [M][K]
  int M, K, G;
  int tiles, tilesets;
  int S;    // waves of a wave-row splitting the groups
  int GS;   // groups per wave (ceil(G / S))
  int y_f16;
};

template <int FMT, int R>
struct WUnit {
  static constexpr int WPG = FMT == 1 ? 1 : 2;  // packed words per lane per tile and group
  uint32_t w[R][WPG];
  uint32_t s[R];   // FP16 scale bits
  u4_t x[4];       // A operand of the four k-steps
};

// Per tile set: the tile starts in both planes (uniform), resolved once per
// set (tiles past the launch resolve to the last tile; their sums are never
// stored).
template <int R>
struct WTiles {
  const uint8_t *w[R];
  const uint16_t *s[R];
  int rt[R];  // rows of each tile (16 but in a matrix's last tile)
};

template <int FMT, int R>
__device__ __forceinline__ void resolve_wtiles(const WideParams &p, WTiles<R> &ts, int t0) {
  const int64_t unit = FMT == 1 ? 16 : 32;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const TileRef tr = tile_ref(p.ms, uni(min(t0 + r, p.tiles - 1)));
    const int RT = uni(min(16, tr.N - 16 * tr.t));
    ts.w[r] = tr.W + 16 * (int64_t)tr.t * p.G * unit;
    ts.s[r] = tr.Sc + 16 * (int64_t)tr.t * p.G;
    ts.rt[r] = RT;
  }
}

// Loads of one unit (group g of the tile set), without branches around them
// and without touching the loaded values: a divergent branch around a load,
// or a value used at once, makes the compiler wait for every load in flight
// (the wait counts are in issue order).  Units outside the sequence re-read
// group 0.  Lanes of rows past a ragged tile, and of token rows past M, read
// row 0 / token 0 again: an A row (token) or B column (row) only feeds its
// own output, and those outputs are never stored.
template <int FMT, int R>
__device__ __forceinline__ void load_wunit(const WideParams &p, const WTiles<R> &ts, WUnit<FMT, R> &u, int g) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const uint16_t *xr = p.X + (j < p.M ? (int64_t)j * p.K : 0) + 128 * g + 8 * q;
#pragma unroll
  for (int s = 0; s < 4; ++s) u.x[s] = *reinterpret_cast<const u4_t *>(xr + 32 * s);
  const int c = g >> 2, gc = g & 3;
  const int Gc = uni(min(4, p.G - 4 * c));
  const int64_t unit = FMT == 1 ? 16 : 32;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int RT = ts.rt[r];
    const int jj = min(j, RT - 1);
    const uint32_t *blk = reinterpret_cast<const uint32_t *>(ts.w[r] + (int64_t)RT * 4 * c * unit);
    if constexpr (FMT == 1) {
      u.w[r][0] = __builtin_nontemporal_load(blk + (q * RT + jj) * Gc + gc);
    } else {
      const int hh = gc >> 1, Gh = min(2, Gc - 2 * hh);
      const u2_t w = __builtin_nontemporal_load(
          reinterpret_cast<const u2_t *>(blk + RT * 16 * hh + ((q * RT + jj) * Gh + (gc - 2 * hh)) * 2));
      u.w[r][0] = w.x;
      u.w[r][1] = w.y;
    }
    u.s[r] = ts.s[r][RT * 4 * c + jj * Gc + gc];  // plane B: chunk c, row jj
  }
}

template <int FMT, bool BF, int R>
__device__ __forceinline__ void compute_wunit(const WUnit<FMT, R> &u, float (&yacc)[R][4]) {
  f4_t acc[R];
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      u4_t b;
      if constexpr (FMT == 1) b = q1_operand_pm1<BF>(u.w[r][0], s);
      else b = tq2_operand(u.w[r][s >> 1], s);
      acc[r] = s == 0 ? mfma16x16x32_zero<BF>(u.x[s], b) : mfma16x16x32<BF>(u.x[s], b, acc[r]);
    }
  }
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const float sc = half_to_float(uint16_t(u.s[r]));
#pragma unroll
    for (int e = 0; e < 4; ++e) yacc[r][e] = fmaf(sc, acc[r][e], yacc[r][e]);
  }
}

template <int FMT, int R>
__device__ __forceinline__ void store_wide(const WideParams &p, int t0, const float (&yacc)[R][4]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const float mul = FMT == 1 ? 1.f : 0.5f;  // ternary operands carry 2t
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (t0 + r >= p.tiles) continue;
    const TileRef tr = tile_ref(p.ms, t0 + r);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * q + e;
      if (m < p.M) store_y(tr, j, m, yacc[r][e] * mul, p.y_f16);
    }
  }
}

// The 8 waves of a workgroup form P = 8 / S wave-rows; wave s of a wave-row
// takes groups [s GS, (s + 1) GS) of each of its tile sets.  Wave-row i of
// workgroup b handles tile sets b + gridDim.x (i + P it), it = 0, 1, ...
// Every wave walks the same number of units (missing ones are skipped
// without loads), so the per-tile-set barrier of the K split is reached by
// all waves.
template <int FMT, bool BF, int R, int D>
__global__ void __launch_bounds__(kThreads, 2) gemv_wide_kernel(WideParams p) {
  __shared__ float red[kWaves * R * 4 * 64];
  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int S = uni(p.S), P = kWaves / S;
  const int pr = uni(wave / S), s = uni(wave - pr * S);
  const int rows_total = gridDim.x * P;
  const int my_row = pr * gridDim.x + blockIdx.x;
  const int iters = (p.tilesets + rows_total - 1) / rows_total;
  const int GS = uni(p.GS);
  const int total = uni(iters * GS);
  const int g_begin = s * GS;

  auto tile0 = [&](int i) { return ((i / GS) * rows_total + my_row) * R; };
  auto group = [&](int i) { return g_begin + i % GS; };
  auto valid = [&](int i) { return (i / GS) * rows_total + my_row < p.tilesets && group(i) < p.G; };

  // The load side walks (tile set, group) with its own cursor and resolves
  // the tile addresses when it enters a tile set.
  int ld_i = 0, ld_k = 0;
  WTiles<R> lts;
  resolve_wtiles<FMT, R>(p, lts, uni(tile0(0)));
  auto load = [&](WUnit<FMT, R> &u) {
    const bool v = ld_i < total && valid(ld_i);
    load_wunit<FMT, R>(p, lts, u, uni(v ? group(ld_i) : 0));
    ++ld_i;
    if (++ld_k == GS) {
      ld_k = 0;
      resolve_wtiles<FMT, R>(p, lts, uni(tile0(ld_i)));
    }
  };

  WUnit<FMT, R> ring[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) load(ring[d]);

  float yacc[R][4];
  for (int i0 = 0; i0 < total; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      // Every step issues its loads and none leaves the loop early, so the
      // wait before a unit's MFMAs covers that unit only.
      load(ring[(d + D - 1) % D]);
      if (i >= total) continue;
      const int k = i % GS;
      if (k == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) yacc[r][e] = 0.f;
      }
      if (valid(i)) compute_wunit<FMT, BF, R>(ring[d], yacc);
      if (k == GS - 1) {
        const int t0 = uni(tile0(i));
        const bool ts_ok = (i / GS) * rows_total + my_row < p.tilesets;
        if (S == 1) {
          if (ts_ok) store_wide<FMT, R>(p, t0, yacc);
        } else {
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < 4; ++e) red[((wave * R + r) * 4 + e) * 64 + lane] = yacc[r][e];
          lds_barrier();
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
            store_wide<FMT, R>(p, t0, tot);
          }
          lds_barrier();
        }
      }
    }
  }
}

// Plan: the (S, grid) with the smallest per-wave work (tile sets per
// wave-row x R x groups per wave), with a small charge for the K-split
// barrier.
template <class Kern>
double plan_wide(const LaunchArgs &a, int R, Kern kernel, WideParams &p, int &grid) {
  p = WideParams{};
  p.ms = mat_set(a);
  p.X = a.X;
  p.M = int(a.M); p.K = int(a.K); p.G = int(a.K / kGroup);
  p.tiles = int((a.N + 15) / 16);
  p.tilesets = (p.tiles + R - 1) / R;
  p.y_f16 = a.y_f16;
  const int slots = num_cus() * resident_blocks(reinterpret_cast<const void *>(kernel), kThreads, 0);
  double best = 1e300;
  WideParams bp = p;
  int bgrid = 1;
  for (int S = 1; S <= 8; S *= 2) {
    if (S > 1 && S > p.G) break;
    const int P = kWaves / S;
    const int g = max(1, min((p.tilesets + P - 1) / P, slots));
    const int64_t rows = (int64_t)g * P;
    const int GS = (p.G + S - 1) / S;
    const double cost = double((p.tilesets + rows - 1) / rows) * R * GS * (S > 1 ? 1.05 : 1.0);
    if (cost < best) {
      best = cost;
      bp = p;
      bp.S = S;
      bp.GS = GS;
      bgrid = g;
    }
  }
  p = bp;
  grid = bgrid;
  return best;
}

template <int FMT, bool BF>
hipError_t launch_wide_t(const LaunchArgs &a) {
  constexpr int D = 3;
  WideParams p1, p2;
  int g1, g2;
  const double c1 = plan_wide(a, 2, &gemv_wide_kernel<FMT, BF, 2, D>, p1, g1);
  const double c2 = plan_wide(a, 4, &gemv_wide_kernel<FMT, BF, 4, D>, p2, g2);
  if (a.plan) {
    const bool two = c1 <= c2 * 1.1;
    const WideParams &p = two ? p1 : p2;
    lowbit_plan &o = plan_record(a, LOWBIT_KERNEL_GEMV_WIDE, two ? g1 : g2, kThreads, 0);
    o.token_slots = 16;
    o.operands = BF ? LOWBIT_OPERANDS_BF16 : LOWBIT_OPERANDS_F16;
    o.tiles_per_wave = two ? 2 : 4;
    o.ring = D;
    o.waves_per_tile = p.S;
    o.groups_per_range = p.GS;
    return hipSuccess;
  }
  if (c1 <= c2 * 1.1)
    hipLaunchKernelGGL((gemv_wide_kernel<FMT, BF, 2, D>), dim3(g1), dim3(kThreads), 0, a.stream, p1);
  else
    hipLaunchKernelGGL((gemv_wide_kernel<FMT, BF, 4, D>), dim3(g2), dim3(kThreads), 0, a.stream, p2);
  return hipGetLastError();
}

}  // namespace

hipError_t launch_gemv_wide(const LaunchArgs &a) {
  if (a.fmt == 1) return a.x_bf16 ? launch_wide_t<1, true>(a) : launch_wide_t<1, false>(a);
  return a.x_bf16 ? launch_wide_t<2, true>(a) : launch_wide_t<2, false>(a);
}

}  // namespace lowbit
