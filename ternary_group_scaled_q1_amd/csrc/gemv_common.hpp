// Pieces shared by the GEMV kernels: wave-uniform values, the per-lane unit
// of packed weights (R row tiles x one chunk of 4 groups in device layout v2)
// and its branch-free load.
#pragma once
#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {
namespace {

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// The matrices of one launch as the kernels see them: row tiles of all of
// them are numbered one after the other (each matrix starts a new tile), so
// a launch over several matrices that share x walks one tile range.
struct MatSet {
  const uint8_t *W[kMaxMats];   // plane A
  const uint16_t *Sc[kMaxMats];  // plane B: FP16 scales (unit order, layout.hpp)
  void *Y[kMaxMats];             // [M][N]
  int N[kMaxMats];
  int tile_end[kMaxMats];        // tiles of matrices 0..i; the total past the last
};

inline MatSet mat_set(const LaunchArgs &a) {
  MatSet m{};
  int end = 0;
  for (int i = 0; i < kMaxMats; ++i) {
    const int k = i < a.nmat ? i : a.nmat - 1;
    m.W[i] = a.Ws[k];
    m.Sc[i] = reinterpret_cast<const uint16_t *>(a.Ws[k] + plane_a_bytes(a.fmt, a.Ns[k], a.K));
    m.Y[i] = a.Ys[k];
    m.N[i] = int(a.Ns[k]);
    if (i < a.nmat) end += int((a.Ns[k] + 15) / 16);
    m.tile_end[i] = end;
  }
  return m;
}

// Matrix and local tile of launch tile vt (wave-uniform: scalar selects).
struct TileRef {
  const uint8_t *W;
  const uint16_t *Sc;
  void *Y;
  int N, t;
};

// Each field read passes through readfirstlane before the selects: a select
// between two fields read straight from the parameter block would be folded
// into one load at a computed offset, which forces a copy of the whole block
// into scratch memory.  The rebuilt address is made a global-memory pointer
// first and only then a generic one: from a plain integer the compiler could
// not tell global memory from LDS and would emit flat loads, whose waits
// also cover every LDS access (each wait then drains all loads in flight).
template <class T>
__device__ __forceinline__ T *uni_ptr(T *ptr) {
  const uint64_t v = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = __builtin_amdgcn_readfirstlane(uint32_t(v));
  const uint32_t hi = __builtin_amdgcn_readfirstlane(uint32_t(v >> 32));
  using GT = __attribute__((address_space(1))) T;
  GT *g = (GT *)((uint64_t(hi) << 32) | lo);
  return (T *)g;
}

__device__ __forceinline__ TileRef tile_ref(const MatSet &m, int vt) {
  TileRef r{uni_ptr(m.W[0]), uni_ptr(m.Sc[0]), uni_ptr(m.Y[0]), uni(m.N[0]), vt};
#pragma unroll
  for (int i = 1; i < kMaxMats; ++i) {
    const int e = uni(m.tile_end[i - 1]);
    const bool c = vt >= e;
    const uint8_t *w = uni_ptr(m.W[i]);
    const uint16_t *sc = uni_ptr(m.Sc[i]);
    void *y = uni_ptr(m.Y[i]);
    const int n = uni(m.N[i]);
    r.W = c ? w : r.W;
    r.Sc = c ? sc : r.Sc;
    r.Y = c ? y : r.Y;
    r.N = c ? n : r.N;
    r.t = c ? vt - e : r.t;
  }
  return r;
}

// Stores value v of token m at row 16 t + j of the tile's matrix (rows past
// the matrix are skipped).
__device__ __forceinline__ void store_y(const TileRef &tr, int j, int m, float v, bool y_f16) {
  const int n = 16 * tr.t + j;
  if (n >= tr.N) return;
  if (y_f16) reinterpret_cast<uint16_t *>(tr.Y)[(int64_t)m * tr.N + n] = float_to_half_rne(v);
  else reinterpret_cast<float *>(tr.Y)[(int64_t)m * tr.N + n] = v;
}

// One A row of a group in the fp8 x fp4 path's LDS staging: 128 bytes of
// pieces in lane order plus 16 bytes that spread the rows over the LDS banks.
constexpr int kRowBytes = 144;

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
// would drain the prefetch ring.  Units that are not valid, and tiles past
// the launch, re-read a valid unit instead of zeroing the registers: their
// values are never used (no MFMA for invalid units, no store past the last
// tile), and the registers of a unit in flight are then written by its own
// loads only.  P provides ms (the matrices), G and tiles (tiles of the
// launch).
template <int FMT, int R, class P>
__device__ __forceinline__ void load_unit(const P &p, Unit<FMT, R> &u, int t0, int c, bool valid) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  const int64_t unit = FMT == 1 ? 16 : 32;
  c = valid ? c : 0;
  t0 = valid ? t0 : 0;
  const int Gc = uni(min(4, p.G - 4 * c));
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const TileRef tr = tile_ref(p.ms, uni(min(t0 + r, p.tiles - 1)));
    const int RT = uni(min(16, tr.N - 16 * tr.t));
    const uint8_t *blk = tr.W + 16 * (int64_t)tr.t * p.G * unit + (int64_t)RT * 4 * c * unit;
    // The unit's scales: 16 T G + RT 4 c, row j at j Gc (plane B).
    const uint16_t *sblk = tr.Sc + 16 * (int64_t)tr.t * p.G + RT * 4 * c;
    if (RT == 16 && Gc == 4) {  // wave-uniform fast path
      const u4_t v0 = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(blk) + lane);
      u.w[r][0] = v0.x; u.w[r][1] = v0.y; u.w[r][2] = v0.z; u.w[r][3] = v0.w;
      if constexpr (FMT == 2) {
        const u4_t v1 = __builtin_nontemporal_load(reinterpret_cast<const u4_t *>(blk + 1024) + lane);
        u.w[r][4] = v1.x; u.w[r][5] = v1.y; u.w[r][6] = v1.z; u.w[r][7] = v1.w;
      }
      const u2_t sv = *reinterpret_cast<const u2_t *>(sblk + 4 * j);
      u.s[r][0] = sv.x; u.s[r][1] = sv.y;
    } else {
      const bool row_ok = j < RT;
      const int jj = min(j, RT - 1);
      const uint32_t *base = reinterpret_cast<const uint32_t *>(blk);
      const uint16_t *srow = sblk + jj * Gc;
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

// Addresses of the R row tiles of one tile set, resolved once per set rather
// than once per unit: the (uniform) start of each tile's packed block and
// each lane's scales in the tile's first chunk.  Tiles past the launch
// resolve to the last tile; their sums are never stored.
template <int R>
struct TileSet {
  const uint8_t *w[R];
  const uint16_t *s[R];
};

template <int FMT, int R, class P>
__device__ __forceinline__ void resolve_tiles(const P &p, TileSet<R> &ts, int t0) {
  const int j = threadIdx.x & 15;
  constexpr int64_t unit = FMT == 1 ? 16 : 32;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const TileRef tr = tile_ref(p.ms, uni(min(t0 + r, p.tiles - 1)));
    ts.w[r] = tr.W + 16 * (int64_t)tr.t * p.G * unit;
    ts.s[r] = tr.Sc + 16 * (int64_t)tr.t * p.G + 4 * j;
  }
}

// Unit (tile set, chunk c) when every tile has 16 rows and every chunk 4
// groups: one 16-byte load per lane and 1 KB (tq2: two, 2 KB) per tile, at a
// fixed stride per chunk, plus the lane's 4 scales.
template <int FMT, int R>
__device__ __forceinline__ void load_full(const TileSet<R> &ts, Unit<FMT, R> &u, int c) {
  const int lane = threadIdx.x & 63;
  constexpr int64_t cb = FMT == 1 ? 1024 : 2048;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    const u4_t *wp = reinterpret_cast<const u4_t *>(ts.w[r] + c * cb) + lane;
    const u4_t v0 = __builtin_nontemporal_load(wp);
    u.w[r][0] = v0.x; u.w[r][1] = v0.y; u.w[r][2] = v0.z; u.w[r][3] = v0.w;
    if constexpr (FMT == 2) {
      const u4_t v1 = __builtin_nontemporal_load(wp + 64);
      u.w[r][4] = v1.x; u.w[r][5] = v1.y; u.w[r][6] = v1.z; u.w[r][7] = v1.w;
    }
    const u2_t sv = *reinterpret_cast<const u2_t *>(ts.s[r] + 64 * c);
    u.s[r][0] = sv.x; u.s[r][1] = sv.y;
  }
}

}  // namespace
}  // namespace lowbit
