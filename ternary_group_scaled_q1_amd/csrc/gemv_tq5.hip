// Decode GEMV for Ternary g128 at 5 trits per byte (tq5), up to 16 tokens:
// Y[m][n] = sum_k X[m][k] t[n][k] s[n][k/128].
//
// Base-3 packing stores 5 trits in a byte (cnblogs.com page, section 2.4),
// 1.725 bits per weight against 2.125 for 2-bit slots, so the same HBM rate
// streams 23% more weights.  In device layout v2 a row is cut into 640-trit
// segments (5 groups): byte w = 8u + e of lane (q, j)'s 32 segment bytes holds
// the weight at in-group offset 32u + 8q + e of all five groups, digit i for
// group i.  A unit of work is R row tiles x one segment: per tile a lane loads
// its 32 bytes (two 16-byte loads; a full tile's segment is 2 KB contiguous)
// and the rows' five FP16 scales, turns each pair of bytes into one word of
// five (sign, non-zero) bit pairs through a 243-entry LDS table (bits 15-2i /
// 14-2i hold trit i of both bytes), and one shift and one AND then give the
// exact 2t bf16/f16 operand pair of group i.  As in the other decode kernels
// the products run on v_mfma_f32_16x16x32 (x as A: lane 16q + j reads 8
// values of token j), each group fills a fresh fp32 tile that is added as
// s * tile, and no dense weight tensor exists (aberweb.com page, section
// 4.1).
//
// The activations are read straight into registers, one group ahead of the
// MFMAs that use them (x is small and shared by every workgroup, so the L2
// and the CU's L1 serve it).  A segment's raw bytes arrive one unit ahead.
// The 8 waves of a workgroup form wave-rows of S waves that split the
// segments; their partial sums are added through LDS in a fixed order.  The
// tail of a row (K mod 640 trits, stored row-major) takes a slow per-weight
// path; it is at most 4 of every 5 groups of one segment.
#include "device.hpp"
#include "gemv_common.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

constexpr int kT5Waves = 8;
constexpr int kT5Threads = 64 * kT5Waves;

struct T5Params {
  MatSet ms;          // the matrices (row tiles numbered across them)
  const uint16_t *X;  // [M][K]
  int M, K, G;
  int tiles, tilesets;
  int nseg;           // segments per row (full ones, plus one for a tail)
  int s_full, b_tail, rowbytes;
  int S;              // waves of a wave-row splitting the segments
  int SS;             // segments per wave (ceil(nseg / S))
  int y_f16;
};

// One token (the decode case) with x staged in LDS: x[0][0..K) as is, then
// a zero cell that the lanes of token slots 1..15 read.
inline int t5_xlds_bytes(int64_t K) { return int(K * 2 + 16); }

// Raw segment bytes and scales of R tiles for one lane.
template <int R>
struct T5Unit {
  u4_t a[R], b[R];    // bytes 0..15 and 16..31 of the lane's segment bytes
  uint16_t s[R][5];   // FP16 scales of the segment's groups (0 past K)
};

// Branch-free loads (ragged tiles clamp addresses and zero values); tail and
// invalid units load nothing into a / b.
template <int R>
__device__ __forceinline__ void t5_load(const T5Params &p, T5Unit<R> &u, int t0, int seg, bool valid) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const u4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int t = uni(t0 + r);
    u.a[r] = z;
    u.b[r] = z;
#pragma unroll
    for (int i = 0; i < 5; ++i) u.s[r][i] = 0;
    if (!valid || t >= p.tiles) continue;  // wave-uniform
    const TileRef tr = tile_ref(p.ms, t);
    const int RT = uni(min(16, tr.N - 16 * tr.t));
    const bool row_ok = j < RT;
    const int jj = min(j, RT - 1);
    const uint8_t *tb = tr.W + 16 * (int64_t)tr.t * p.rowbytes;
    if (seg < p.s_full) {  // wave-uniform
      const uint8_t *sb = tb + (int64_t)RT * 128 * seg + (q * RT + jj) * 16;
      const u4_t va = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(sb));
      const u4_t vb = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(sb + RT * 64));
      u.a[r] = row_ok ? va : z;
      u.b[r] = row_ok ? vb : z;
    }
    // Plane B: the segment's scales start at 16 T G + RT 5 seg, row jj at jj Gs.
    const int Gs = uni(min(5, p.G - 5 * seg));
    const uint16_t *srow = tr.Sc + 16 * (int64_t)tr.t * p.G + RT * 5 * seg + jj * Gs;
#pragma unroll
    for (int i = 0; i < 5; ++i) {
      const uint16_t v = srow[min(i, Gs - 1)];
      u.s[r][i] = row_ok && i < Gs ? v : uint16_t(0);
    }
  }
}

// x fragment of group g (4 k-steps): lane 16q + j holds x[j][128 g + 32 u + 8 q .. + 8].
__device__ __forceinline__ void t5_load_x(const T5Params &p, u4_t (&x)[4], int g, bool valid) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const bool tok = valid && j < p.M;
  const uint16_t *xr = p.X + (tok ? (int64_t)j * p.K + 128 * g : 0) + 8 * q;
  const u4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const u4_t v = *reinterpret_cast<const u4_t *>(xr + 32 * u);
    x[u] = tok ? v : z;
  }
}

// The same from the LDS copy of x (one token): cell k / 8 for lanes of token
// 0, the zero cell past K for the others.
__device__ __forceinline__ void t5_lds_x(const T5Params &p, const char *xl, u4_t (&x)[4], int g) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const int base = j == 0 ? (128 * g + 8 * q) * 2 : p.K * 2;
  const int step = j == 0 ? 64 : 0;
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const u4_t *>(xl + base + step * u);
}

// (sign, non-zero) words of the lane's segment bytes: d[u * 4 + p] holds the
// five pairs of bytes 8u + 2p (low half) and 8u + 2p + 1 (high half).
__device__ __forceinline__ void t5_decode(const u4_t &a, const u4_t &b, const uint16_t *lut, uint32_t (&d)[16]) {
  const uint32_t wds[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
#pragma unroll
  for (int w = 0; w < 16; ++w) {
    const uint32_t word = wds[w >> 1];
    const uint32_t b0 = (word >> (16 * (w & 1))) & 0xFF;
    const uint32_t b1 = (word >> (16 * (w & 1) + 8)) & 0xFF;
    d[w] = uint32_t(lut[b0]) | (uint32_t(lut[b1]) << 16);
  }
}

// Tail segment (row-major bytes, B = b_tail per row): the 2t operand of
// k-step u, group i of the tail, for this lane's row.
__device__ __forceinline__ u4_t t5_tail_operand(const T5Params &p, const TileRef &tr, int i, int u) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const int RT = min(16, tr.N - 16 * tr.t);
  const int jj = min(j, RT - 1);
  const uint8_t *rb = tr.W + 16 * (int64_t)tr.t * p.rowbytes + (int64_t)RT * 128 * p.s_full + (int64_t)jj * p.b_tail;
  uint32_t h[8];
#pragma unroll
  for (int e = 0; e < 8; ++e) {
    const int kt = 128 * i + 32 * u + 8 * q + e;
    int v = rb[kt % p.b_tail];
    for (int t = kt / p.b_tail; t > 0; --t) v /= 3;
    const int dgt = v % 3;
    h[e] = dgt == 1 ? 0u : (dgt == 2 ? 0x4000u : 0xC000u);
  }
  u4_t o;
  o.x = h[0] | (h[1] << 16);
  o.y = h[2] | (h[3] << 16);
  o.z = h[4] | (h[5] << 16);
  o.w = h[6] | (h[7] << 16);
  return o;
}

template <int R>
__device__ __forceinline__ void t5_store(const T5Params &p, int t0, const float (&yacc)[R][4]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (t0 + r >= p.tiles) continue;
    const TileRef tr = tile_ref(p.ms, t0 + r);
#pragma unroll
    for (int e = 0; e < 4; ++e) {
      const int m = 4 * q + e;
      if (m < p.M) store_y(tr, j, m, yacc[r][e] * 0.5f, p.y_f16);  // operands carry 2t
    }
  }
}

// XL: one token, x staged in LDS (read right before its MFMAs) and the
// weights three units deep; else x one group ahead in registers and the
// weights two units deep.
template <bool BF, int R, bool XL>
__global__ void __launch_bounds__(kT5Threads, 2) gemv_tq5_kernel(T5Params p) {
  __shared__ uint16_t lut[256];
  __shared__ float red[kT5Waves * R * 4 * 64];
  extern __shared__ __align__(16) char xl[];
  if constexpr (XL) {
    for (int i = threadIdx.x; i < p.K / 8; i += kT5Threads)
      reinterpret_cast<u4_t *>(xl)[i] = reinterpret_cast<const u4_t *>(p.X)[i];
    if (threadIdx.x == 0) *reinterpret_cast<u4_t *>(xl + p.K * 2) = u4_t{0u, 0u, 0u, 0u};
  }
  for (int v = threadIdx.x; v < 256; v += kT5Threads) {
    uint32_t f = 0;
    int dgt = v;
    for (int i = 0; i < 5; ++i) {
      const int di = dgt % 3;
      dgt /= 3;
      f |= (uint32_t(di == 0) << (15 - 2 * i)) | (uint32_t(di != 1) << (14 - 2 * i));
    }
    lut[v] = uint16_t(v < 243 ? f : 0);
  }
  lds_barrier();

  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int S = uni(p.S), P = kT5Waves / S;
  const int pr = uni(wave / S), s = uni(wave - pr * S);
  const int rows_total = gridDim.x * P;
  const int my_row = pr * gridDim.x + blockIdx.x;
  const int iters = (p.tilesets + rows_total - 1) / rows_total;
  const int SS = uni(p.SS);
  const int total = uni(iters * SS);
  const int seg0 = s * SS;

  auto tile0 = [&](int i) { return ((i / SS) * rows_total + my_row) * R; };
  auto segment = [&](int i) { return seg0 + i % SS; };
  auto valid = [&](int i) { return i < total && (i / SS) * rows_total + my_row < p.tilesets && segment(i) < p.nseg; };

  T5Unit<R> cur, nxt, nx2;
  t5_load<R>(p, cur, uni(tile0(0)), uni(segment(0)), valid(0));
  if constexpr (XL) t5_load<R>(p, nxt, uni(tile0(1)), uni(segment(1)), valid(1));
  u4_t xc[4], xn[4];
  if constexpr (!XL) t5_load_x(p, xc, 5 * segment(0), valid(0));

  float yacc[R][4];
  for (int i = 0; i < total; ++i) {
    const bool vi = valid(i);
    const int seg = uni(segment(i));
    const int t0 = uni(tile0(i));
    // The weights of unit i + 1 (XL: i + 2) go out before this one is worked on.
    if constexpr (XL) t5_load<R>(p, nx2, uni(tile0(i + 2)), uni(segment(i + 2)), valid(i + 2));
    else t5_load<R>(p, nxt, uni(tile0(i + 1)), uni(segment(i + 1)), valid(i + 1));
    if (i % SS == 0) {
#pragma unroll
      for (int r = 0; r < R; ++r)
#pragma unroll
        for (int e = 0; e < 4; ++e) yacc[r][e] = 0.f;
    }
    if (vi) {  // wave-uniform
      const int ng = uni(min(5, p.G - 5 * seg));
      const int gnext = 5 * uni(segment(i + 1));
      const bool vnext = valid(i + 1);
      if (seg < p.s_full) {  // full segment: five groups through the table
        uint32_t d[R][16];
#pragma unroll
        for (int r = 0; r < R; ++r) t5_decode(cur.a[r], cur.b[r], lut, d[r]);
#pragma unroll
        for (int gi = 0; gi < 5; ++gi) {
          // x of the next group (of this segment, else of the next unit).
          if constexpr (XL) t5_lds_x(p, xl, xc, 5 * seg + gi);
          else if (gi < 4) t5_load_x(p, xn, 5 * seg + gi + 1, true);
          else t5_load_x(p, xn, gnext, vnext);
          f4_t acc[R];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
              u4_t bop;
              bop.x = tq5_pair(d[r][4 * u + 0], gi);
              bop.y = tq5_pair(d[r][4 * u + 1], gi);
              bop.z = tq5_pair(d[r][4 * u + 2], gi);
              bop.w = tq5_pair(d[r][4 * u + 3], gi);
              acc[r] = u == 0 ? mfma16x16x32_zero<BF>(xc[u], bop) : mfma16x16x32<BF>(xc[u], bop, acc[r]);
            }
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const float sc = half_to_float(cur.s[r][gi]);
#pragma unroll
            for (int e = 0; e < 4; ++e) yacc[r][e] = fmaf(sc, acc[r][e], yacc[r][e]);
          }
          if constexpr (!XL) {
#pragma unroll
            for (int u = 0; u < 4; ++u) xc[u] = xn[u];
          }
        }
      } else {  // tail segment: ng < 5 groups, row-major bytes
        for (int gi = 0; gi < ng; ++gi) {
          const int gnx = gi + 1 < ng ? 5 * seg + gi + 1 : gnext;
          if constexpr (XL) t5_lds_x(p, xl, xc, 5 * seg + gi);
          else t5_load_x(p, xn, gnx, gi + 1 < ng ? true : vnext);
          f4_t acc[R];
#pragma unroll
          for (int u = 0; u < 4; ++u) {
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const int t = t0 + r < p.tiles ? t0 + r : 0;
              const u4_t bop = t5_tail_operand(p, tile_ref(p.ms, t), gi, u);
              acc[r] = u == 0 ? mfma16x16x32_zero<BF>(xc[u], bop) : mfma16x16x32<BF>(xc[u], bop, acc[r]);
            }
          }
#pragma unroll
          for (int r = 0; r < R; ++r) {
            const uint16_t sh = gi == 0 ? cur.s[r][0] : gi == 1 ? cur.s[r][1] : gi == 2 ? cur.s[r][2] : cur.s[r][3];
            const float sc = half_to_float(sh);
#pragma unroll
            for (int e = 0; e < 4; ++e) yacc[r][e] = fmaf(sc, acc[r][e], yacc[r][e]);
          }
          if constexpr (!XL) {
#pragma unroll
            for (int u = 0; u < 4; ++u) xc[u] = xn[u];
          }
        }
      }
    } else if constexpr (!XL) {
      t5_load_x(p, xc, 5 * uni(segment(i + 1)), valid(i + 1));
    }
    cur = nxt;
    if constexpr (XL) nxt = nx2;
    if (i % SS == SS - 1) {
      const bool ts_ok = (i / SS) * rows_total + my_row < p.tilesets;
      if (S == 1) {
        if (ts_ok) t5_store<R>(p, t0, yacc);
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
          t5_store<R>(p, t0, tot);
        }
        lds_barrier();
      }
    }
  }
}

// Addresses of the R tiles of one tile set, resolved once per set: the
// tile's start in both planes and the tile's rows (tiles past the launch
// resolve to the last tile; their sums are never stored).
template <int R>
struct T5Tiles {
  const uint8_t *w[R];
  const uint16_t *s[R];
  int rt[R];
};

template <int R>
__device__ __forceinline__ void t5_resolve(const T5Params &p, T5Tiles<R> &ts, int t0) {
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const TileRef tr = tile_ref(p.ms, uni(min(t0 + r, p.tiles - 1)));
    const int RT = uni(min(16, tr.N - 16 * tr.t));
    ts.w[r] = tr.W + 16 * (int64_t)tr.t * p.rowbytes;
    ts.s[r] = tr.Sc + 16 * (int64_t)tr.t * p.G;
    ts.rt[r] = RT;
  }
}

// Loads of unit (tile set, segment seg) with neither branches nor masks, so
// that each step of the ring issues the same loads: the row tail's segment
// (read by the per-weight path) re-reads the last full segment, or the
// tile's first bytes when a row has no full segment (the scales plane
// follows the packed bytes, so 32 bytes from a tile's start stay inside the
// blob); rows past a ragged tile re-read its last row, groups past K the
// segment's last scale and units past the row its last segment's scales.
// None of those values reaches a stored output.
template <int R>
__device__ __forceinline__ void t5_load_ts(const T5Params &p, const T5Tiles<R> &ts, T5Unit<R> &u, int seg) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const int sf = uni(max(min(seg, p.s_full - 1), 0));
  const int ss = uni(max(min(seg, p.nseg - 1), 0));  // segment of the scales
  const int Gs = uni(min(5, p.G - 5 * ss));
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const int RT = ts.rt[r];
    const int jj = min(j, RT - 1);
    const uint8_t *sb = p.s_full > 0 ? ts.w[r] + (int64_t)RT * 128 * sf + (q * RT + jj) * 16 : ts.w[r];
    const int hb = p.s_full > 0 ? RT * 64 : 0;
    u.a[r] = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(sb));
    u.b[r] = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(sb + hb));
#pragma unroll
    for (int i = 0; i < 5; ++i) u.s[r][i] = ts.s[r][RT * 5 * ss + jj * Gs + min(i, Gs - 1)];
  }
}

// One token with x staged in LDS: the units of a wave form a ring of three,
// stepped by compile-time slots (no register moves between units), every
// step issues its loads and none leaves the loop early, so the wait before a
// unit's MFMAs covers that unit only.  The x of the whole K is loaded into
// registers before the first weights and written to LDS after them.
template <bool BF, int R>
__global__ void __launch_bounds__(kT5Threads, 2) gemv_tq5_one_kernel(T5Params p) {
  constexpr int D = 3;
  constexpr int kXPre = 4;  // x cells per thread loaded before the weights
  __shared__ uint16_t lut[256];
  __shared__ float red[kT5Waves * R * 4 * 64];
  extern __shared__ __align__(16) char xl[];

  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int S = uni(p.S), P = kT5Waves / S;
  const int pr = uni(wave / S), s = uni(wave - pr * S);
  const int rows_total = gridDim.x * P;
  const int my_row = pr * gridDim.x + blockIdx.x;
  const int iters = (p.tilesets + rows_total - 1) / rows_total;
  const int SS = uni(p.SS);
  const int total = uni(iters * SS);
  const int seg0 = s * SS;

  auto tile0 = [&](int i) { return ((i / SS) * rows_total + my_row) * R; };
  auto segment = [&](int i) { return seg0 + i % SS; };
  auto valid = [&](int i) { return i < total && (i / SS) * rows_total + my_row < p.tilesets && segment(i) < p.nseg; };

  // x cells (8 values each) of the first kXPre passes over the workgroup.
  const int cells = p.K / 8;
  u4_t xpre[kXPre];
#pragma unroll
  for (int c = 0; c < kXPre; ++c)
    xpre[c] = reinterpret_cast<const u4_t *>(p.X)[min(int(threadIdx.x) + c * kT5Threads, cells - 1)];

  // The load side: its cursor and the tile set it reads.
  int ld_i = 0, ld_k = 0;
  T5Tiles<R> lts;
  t5_resolve<R>(p, lts, uni(tile0(0)));
  auto load = [&](T5Unit<R> &u) {
    const bool v = valid(ld_i);
    t5_load_ts<R>(p, lts, u, uni(v ? segment(ld_i) : seg0));
    ++ld_i;
    if (++ld_k == SS) {
      ld_k = 0;
      t5_resolve<R>(p, lts, uni(tile0(ld_i)));
    }
  };
  T5Unit<R> ring[D];
#pragma unroll
  for (int d = 0; d < D - 1; ++d) load(ring[d]);

#pragma unroll
  for (int c = 0; c < kXPre; ++c) {
    const int cell = int(threadIdx.x) + c * kT5Threads;
    if (cell < cells) reinterpret_cast<u4_t *>(xl)[cell] = xpre[c];
  }
  for (int cell = int(threadIdx.x) + kXPre * kT5Threads; cell < cells; cell += kT5Threads)
    reinterpret_cast<u4_t *>(xl)[cell] = reinterpret_cast<const u4_t *>(p.X)[cell];
  if (threadIdx.x == 0) *reinterpret_cast<u4_t *>(xl + p.K * 2) = u4_t{0u, 0u, 0u, 0u};
  for (int v = threadIdx.x; v < 256; v += kT5Threads) {
    uint32_t f = 0;
    int dgt = v;
    for (int i = 0; i < 5; ++i) {
      const int di = dgt % 3;
      dgt /= 3;
      f |= (uint32_t(di == 0) << (15 - 2 * i)) | (uint32_t(di != 1) << (14 - 2 * i));
    }
    lut[v] = uint16_t(v < 243 ? f : 0);
  }
  lds_barrier();

  float yacc[R][4];
  for (int i0 = 0; i0 < total; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      load(ring[(d + D - 1) % D]);
      if (i >= total) continue;
      const T5Unit<R> &cur = ring[d];
      const int seg = uni(segment(i));
      const int t0 = uni(tile0(i));
      if (i % SS == 0) {
#pragma unroll
        for (int r = 0; r < R; ++r)
#pragma unroll
          for (int e = 0; e < 4; ++e) yacc[r][e] = 0.f;
      }
      if (valid(i)) {  // wave-uniform
        const int ng = uni(min(5, p.G - 5 * seg));
        u4_t xc[4];
        if (seg < p.s_full) {  // full segment: five groups through the table
          uint32_t dd[R][16];
#pragma unroll
          for (int r = 0; r < R; ++r) t5_decode(cur.a[r], cur.b[r], lut, dd[r]);
#pragma unroll
          for (int gi = 0; gi < 5; ++gi) {
            t5_lds_x(p, xl, xc, 5 * seg + gi);
            f4_t acc[R];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
              for (int r = 0; r < R; ++r) {
                u4_t bop;
                bop.x = tq5_pair(dd[r][4 * u + 0], gi);
                bop.y = tq5_pair(dd[r][4 * u + 1], gi);
                bop.z = tq5_pair(dd[r][4 * u + 2], gi);
                bop.w = tq5_pair(dd[r][4 * u + 3], gi);
                acc[r] = u == 0 ? mfma16x16x32_zero<BF>(xc[u], bop) : mfma16x16x32<BF>(xc[u], bop, acc[r]);
              }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const float sc = half_to_float(cur.s[r][gi]);
#pragma unroll
              for (int e = 0; e < 4; ++e) yacc[r][e] = fmaf(sc, acc[r][e], yacc[r][e]);
            }
          }
        } else {  // tail segment: ng < 5 groups, row-major bytes
          for (int gi = 0; gi < ng; ++gi) {
            t5_lds_x(p, xl, xc, 5 * seg + gi);
            f4_t acc[R];
#pragma unroll
            for (int u = 0; u < 4; ++u) {
#pragma unroll
              for (int r = 0; r < R; ++r) {
                const int t = t0 + r < p.tiles ? t0 + r : 0;
                const u4_t bop = t5_tail_operand(p, tile_ref(p.ms, t), gi, u);
                acc[r] = u == 0 ? mfma16x16x32_zero<BF>(xc[u], bop) : mfma16x16x32<BF>(xc[u], bop, acc[r]);
              }
            }
#pragma unroll
            for (int r = 0; r < R; ++r) {
              const uint16_t sh = gi == 0 ? cur.s[r][0] : gi == 1 ? cur.s[r][1] : gi == 2 ? cur.s[r][2] : cur.s[r][3];
              const float sc = half_to_float(sh);
#pragma unroll
              for (int e = 0; e < 4; ++e) yacc[r][e] = fmaf(sc, acc[r][e], yacc[r][e]);
            }
          }
        }
      }
      if (i % SS == SS - 1) {
        const bool ts_ok = (i / SS) * rows_total + my_row < p.tilesets;
        if (S == 1) {
          if (ts_ok) t5_store<R>(p, t0, yacc);
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
            t5_store<R>(p, t0, tot);
          }
          lds_barrier();
        }
      }
    }
  }
}

// Plan: the (S, grid) with the smallest per-wave work (tile sets per
// wave-row x R x segments per wave), with a small charge for the K split.
template <class Kern>
double plan_tq5(const LaunchArgs &a, int R, Kern kernel, int lds, T5Params &p, int &grid) {
  p = T5Params{};
  p.ms = mat_set(a);
  p.X = a.X;
  p.M = int(a.M); p.K = int(a.K); p.G = int(a.K / kGroup);
  p.tiles = int((a.N + 15) / 16);
  p.tilesets = (p.tiles + R - 1) / R;
  const Tq5Geom g = tq5_geom(a.K);
  p.s_full = int(g.s_full);
  p.b_tail = int(g.b_tail);
  p.rowbytes = int(g.rowbytes);
  p.nseg = p.s_full + (g.L_tail > 0 ? 1 : 0);
  p.y_f16 = a.y_f16;
  const int slots = num_cus() * resident_blocks(reinterpret_cast<const void *>(kernel), kT5Threads, lds);
  double best = 1e300;
  T5Params bp = p;
  int bgrid = 1;
  for (int S = 1; S <= 8; S *= 2) {
    if (S > 1 && S > p.nseg) break;
    const int P = kT5Waves / S;
    const int gsz = max(1, min((p.tilesets + P - 1) / P, slots));
    const int64_t rows = (int64_t)gsz * P;
    const int SS = (p.nseg + S - 1) / S;
    const double cost = double((p.tilesets + rows - 1) / rows) * R * SS * (S > 1 ? 1.05 : 1.0);
    if (cost < best) {
      best = cost;
      bp = p;
      bp.S = S;
      bp.SS = SS;
      bgrid = gsz;
    }
  }
  p = bp;
  grid = bgrid;
  return best;
}

template <bool BF, bool XL>
hipError_t launch_tq5_x(const LaunchArgs &a) {
  T5Params p1, p2;
  int g1, g2;
  const int lds = XL ? t5_xlds_bytes(a.K) : 0;
  const double c1 = plan_tq5(a, 1, &gemv_tq5_kernel<BF, 1, XL>, lds, p1, g1);
  const double c2 = plan_tq5(a, 2, &gemv_tq5_kernel<BF, 2, XL>, lds, p2, g2);
  if (a.plan) {
    const bool one = c1 <= c2 * 1.1;
    const T5Params &p = one ? p1 : p2;
    lowbit_plan &o = plan_record(a, LOWBIT_KERNEL_GEMV_TQ5, one ? g1 : g2, kT5Threads, lds);
    o.token_slots = 16;
    o.operands = BF ? LOWBIT_OPERANDS_BF16 : LOWBIT_OPERANDS_F16;
    o.tiles_per_wave = one ? 1 : 2;
    o.ring = 2;
    o.waves_per_tile = p.S;
    o.groups_per_range = 5 * p.SS;
    return hipSuccess;
  }
  if (c1 <= c2 * 1.1)
    hipLaunchKernelGGL((gemv_tq5_kernel<BF, 1, XL>), dim3(g1), dim3(kT5Threads), lds, a.stream, p1);
  else
    hipLaunchKernelGGL((gemv_tq5_kernel<BF, 2, XL>), dim3(g2), dim3(kT5Threads), lds, a.stream, p2);
  return hipGetLastError();
}

// Plan of the one-token kernel, from timings of the 27B-class decode shapes
// on MI355X (every R, S and 1 or 2 workgroups per CU): one tile per wave and
// two workgroups per CU.  When the tiles fill every wave slot of that grid
// (the LM head) K stays whole; otherwise K is cut over the fewest waves S (a
// power of two, at most 8) that leave each wave at most two of a row's
// segments (gate/up 34816 x 5120: 21.5 us, against 27.4 us for the plan
// that minimised the CU-sharing cost of the other decode kernels, which kept
// K whole and put one workgroup on most CUs; the LM head 65.6 us with K
// whole, 75.7 us cut over 4 waves).
void plan_tq5_one(const LaunchArgs &a, const void *kernel, int lds, T5Params &p, int &grid) {
  p = T5Params{};
  p.ms = mat_set(a);
  p.X = a.X;
  p.M = int(a.M); p.K = int(a.K); p.G = int(a.K / kGroup);
  p.tiles = int((a.N + 15) / 16);
  p.tilesets = p.tiles;  // one tile per wave
  const Tq5Geom g = tq5_geom(a.K);
  p.s_full = int(g.s_full);
  p.b_tail = int(g.b_tail);
  p.rowbytes = int(g.rowbytes);
  p.nseg = p.s_full + (g.L_tail > 0 ? 1 : 0);
  p.y_f16 = a.y_f16;
  const int per_cu = resident_blocks(kernel, kT5Threads, lds);
  const int slots = num_cus() * min(per_cu, 2);  // workgroups resident at once
  int S = 1;
  if (p.tilesets < slots * kT5Waves)
    while (S < 8 && (p.nseg + S - 1) / S > 2) S *= 2;
  p.S = S;
  p.SS = (p.nseg + S - 1) / S;
  const int P = kT5Waves / S;  // tile sets per workgroup pass
  const int want = (p.tilesets + P - 1) / P;
  grid = max(1, min(want, slots));
}

template <bool BF>
hipError_t launch_tq5_one(const LaunchArgs &a) {
  T5Params p;
  int grid;
  const int lds = t5_xlds_bytes(a.K);
  plan_tq5_one(a, reinterpret_cast<const void *>(&gemv_tq5_one_kernel<BF, 1>), lds, p, grid);
  if (a.plan) {
    lowbit_plan &o = plan_record(a, LOWBIT_KERNEL_GEMV_TQ5_ONE, grid, kT5Threads, lds);
    o.token_slots = 1;
    o.operands = BF ? LOWBIT_OPERANDS_BF16 : LOWBIT_OPERANDS_F16;
    o.tiles_per_wave = 1;
    o.ring = 3;
    o.waves_per_tile = p.S;
    o.groups_per_range = 5 * p.SS;
    o.groups_per_pass = p.G;
    return hipSuccess;
  }
  hipLaunchKernelGGL((gemv_tq5_one_kernel<BF, 1>), dim3(grid), dim3(kT5Threads), lds, a.stream, p);
  return hipGetLastError();
}

// One token whose x fits in 64 KB of LDS: staged once per workgroup (the
// ring kernel above); else x read into registers one group ahead.
template <bool BF>
hipError_t launch_tq5_t(const LaunchArgs &a) {
  if (a.M == 1 && t5_xlds_bytes(a.K) <= 64 * 1024) return launch_tq5_one<BF>(a);
  return launch_tq5_x<BF, false>(a);
}

}  // namespace

hipError_t launch_gemv_tq5(const LaunchArgs &a) {
  return a.x_bf16 ? launch_tq5_t<true>(a) : launch_tq5_t<false>(a);
}

}  // namespace lowbit
