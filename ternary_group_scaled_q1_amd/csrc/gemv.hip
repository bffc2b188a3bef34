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
// Two product paths share the work split below:
//  * bf16 x, up to 8 tokens: the weights decode to fp4 (e2m1) and each
//    128-weight group is one scaled 16x16x128 fp8 x fp4 MFMA.  x enters as two
//    exact fp8 (e4m3) pieces per value, x = S (hi + lo), with one power-of-two
//    scale S per token and 32 values (the instruction's E8M0 operand scale):
//    a bf16 value has 8 significant bits and each piece carries 4, so the
//    split is exact unless a value sits more than 2^10 below the largest of
//    its 32 (then the error is below 2^-17 of that largest value).  The A rows
//    are (token, piece) pairs; the two pieces' products are added in fp32.
//    fp16 x at one token takes the same instruction with three pieces
//    (hi, mid, lo: an fp16 value has 11 significant bits), exact for values
//    within 2^6 of their block's largest (split_x_regs_f16).
//  * fp16 x at several tokens, ternary weights, or more than 8 tokens:
//    v_mfma_f32_16x16x32 on exact f16/bf16 operands.
//
// Work split: a workgroup of 8 waves stages x in LDS as [k/8][token][8]
// 16-byte cells, all of K at once when it fits (then the stage is loaded
// once per workgroup) or S chunks at a time.  The waves form P = 8/S
// wave-rows; a wave-row owns R row tiles (16R rows) at a time and its S
// waves split each stage's chunks, adding their partial sums through LDS in
// a fixed order, so results are deterministic.  All control flow that
// decides loads, MFMAs and barriers is wave-uniform.
#include "device.hpp"
#include "gemv_common.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

constexpr int kWaves = 8;
constexpr int kThreads = 64 * kWaves;

struct GemvParams {
  MatSet ms;           // the matrices (row tiles numbered across them)
  const uint16_t *X;   // [M][K]
  int M, K, G;
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

// fp8 x fp4 path: per group, NPC*MP A rows of kRowBytes (gemv_common.hpp),
// then MP*4 E8M0 scale bytes per group.  NPC = pieces per token: two for
// bf16 x, three for fp16 x (one token only).

inline LdsMap lds_map_fp4(int MP, int NPC, int S, int SC, int R, int E) {
  LdsMap m;
  const int groups = 4 * SC;
  m.corr = 0;
  m.x = 0;
  int o = groups * NPC * MP * kRowBytes;
  m.corr = o;  // E8M0 scale bytes
  o += (groups * MP * 4 + 15) / 16 * 16;
  m.red = o;
  if (S > 1) o += kWaves * R * E * 64 * 4;
  m.total = o;
  return m;
}

// x staging runs in two steps, so that the loads of each thread's first
// item go out before the weight prefetch: XFirst holds that item as loaded,
// and the staging pass converts and writes it, then loads and writes any
// further items one by one.  A wait for x counts only the loads issued
// before it, so the weight loads stay in flight while x is converted.
template <bool FP4>
struct XFirst {
  static constexpr int kCells = FP4 ? 1 : 4;  // exact operands: up to 4 passes' cells
  u4_t v[FP4 ? 4 : kCells];
};

// fp8 x fp4 item it: token slot m, group gl of the pass, lane quarter q.
// Items past the pass (m >= MP) and tokens past M read x[0] and stage zeros.
template <int MP>
__device__ __forceinline__ const uint16_t *fp4_item(const GemvParams &p, int it, int c0, int nc, bool &in) {
  const int q = it & 3, rest = it >> 2;
  const int gl = rest % (4 * nc), m = rest / (4 * nc);
  in = m < p.M && 4 * c0 + gl < p.G;
  return p.X + (in ? (int64_t)m * p.K + 128 * (4 * c0 + gl) + 8 * q : 0);
}

template <int MP>
__device__ __forceinline__ void fp4_item_load(const GemvParams &p, int it, int c0, int nc, u4_t (&raw)[4]) {
  bool in;
  const uint16_t *src = fp4_item<MP>(p, it, c0, nc, in);
#pragma unroll
  for (int u = 0; u < 4; ++u) raw[u] = *reinterpret_cast<const u4_t *>(src + 32 * u);
}

// Splits the item's 32 values into A rows 2m (hi) and 2m + 1 (lo) of its
// group (bf16 x, split_x_regs), or 3m, 3m + 1, 3m + 2 (hi, mid, lo: fp16 x,
// split_x_regs_f16), and writes its E8M0 scale byte.  The quarter's values
// sit at hardware k 32q + n; the A operand holds k < 64 in bytes 0..15 and
// k >= 64 in bytes 16..31 of lane quarter (k % 64) / 16, so nibbles 0..15 go
// to lane quarter 2(q % 2) and 16..31 to 2(q % 2) + 1.
template <int FMT, bool BF, int MP>
__device__ __forceinline__ void fp4_item_write(const GemvParams &p, char *lds, int it, int c0, int nc,
                                               const u4_t (&raw)[4]) {
  const int q = it & 3, rest = it >> 2;
  const int gl = rest % (4 * nc), m = rest / (4 * nc);
  bool in;
  fp4_item<MP>(p, it, c0, nc, in);
  const u4_t z = {0u, 0u, 0u, 0u};
  u4_t x[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) x[u] = in ? raw[u] : z;
  const int qa = 2 * (q & 1), half = 16 * (q >> 1);
  if constexpr (BF) {
    XQuarter xq;
    split_x_regs<FMT>(x, xq);
    char *row = lds + p.off_x + (gl * 2 * MP + 2 * m) * kRowBytes;
    *reinterpret_cast<u4_t *>(row + qa * 32 + half) = xq.h0;
    *reinterpret_cast<u4_t *>(row + (qa + 1) * 32 + half) = xq.h1;
    *reinterpret_cast<u4_t *>(row + kRowBytes + qa * 32 + half) = xq.l0;
    *reinterpret_cast<u4_t *>(row + kRowBytes + (qa + 1) * 32 + half) = xq.l1;
    reinterpret_cast<uint8_t *>(lds + p.off_corr)[(gl * MP + m) * 4 + q] = xq.sb;
  } else {
    XQuarter3 xq;
    split_x_regs_f16<FMT>(x, xq);
    char *row = lds + p.off_x + (gl * 3 * MP + 3 * m) * kRowBytes;
    *reinterpret_cast<u4_t *>(row + qa * 32 + half) = xq.h0;
    *reinterpret_cast<u4_t *>(row + (qa + 1) * 32 + half) = xq.h1;
    *reinterpret_cast<u4_t *>(row + kRowBytes + qa * 32 + half) = xq.m0;
    *reinterpret_cast<u4_t *>(row + kRowBytes + (qa + 1) * 32 + half) = xq.m1;
    *reinterpret_cast<u4_t *>(row + 2 * kRowBytes + qa * 32 + half) = xq.l0;
    *reinterpret_cast<u4_t *>(row + 2 * kRowBytes + (qa + 1) * 32 + half) = xq.l1;
    reinterpret_cast<uint8_t *>(lds + p.off_corr)[(gl * MP + m) * 4 + q] = xq.sb;
  }
}

// Stage chunks [c0, c0 + nc) of x for the fp8 x fp4 path: one item per
// (token slot, group, lane quarter); tokens m >= M and groups past K stage as
// zeros.  PRE: the thread's first item was loaded into first.
template <int FMT, bool BF, int MP, bool PRE>
__device__ void stage_fp4(const GemvParams &p, char *lds, int c0, int nc, const XFirst<true> &first) {
  const int items = MP * 4 * nc * 4;
  int it = threadIdx.x;
  if constexpr (PRE) {
    if (it < items) fp4_item_write<FMT, BF, MP>(p, lds, it, c0, nc, first.v);
    it += kThreads;
  }
  for (; it < items; it += kThreads) {
    u4_t raw[4];
    fp4_item_load<MP>(p, it, c0, nc, raw);
    fp4_item_write<FMT, BF, MP>(p, lds, it, c0, nc, raw);
  }
}

// Cell idx of the exact-operand staging: token slot m, k-octet oct.
template <int MTS>
__device__ __forceinline__ const u4_t *x_cell(const GemvParams &p, int idx, int c0, int nc, bool &in) {
  const int m = idx / (nc * 64), oct = idx - m * (nc * 64);
  const int k = c0 * 512 + oct * 8;
  in = idx < MTS * nc * 64 && k < p.K && m < p.M;
  return reinterpret_cast<const u4_t *>(p.X + (in ? (int64_t)m * p.K + k : 0));
}

// Stage chunks [c0, c0 + nc) of x: cell (oct, m) holds x[m][k0 + 8 oct .. + 8] at
// byte off_x + (oct * MTS + m) * 16 (zeros past K and for m >= M).  One thread
// per (group, token slot) also sums the group's activations at k % 4 in {2, 3}:
// the q1 operand feeds those weights as t + 1, so minus that sum is stored in
// corr[group][token] and seeds the group's accumulator.  PRE: the thread's
// first cell was loaded into first.
template <int FMT, bool BF, int MTS, bool PRE>
__device__ void stage_x(const GemvParams &p, char *lds, int c0, int nc, const XFirst<false> &first) {
  uint4 *xl = reinterpret_cast<uint4 *>(lds + p.off_x);
  float *corr = reinterpret_cast<float *>(lds + p.off_corr);
  // One thread per (token slot, k-octet); the 16 octets of a group sit in 16
  // consecutive lanes, which add up the group's correction by shuffles.
  const int cells = MTS * nc * 64;
  for (int base = 0; base < cells; base += kThreads) {
    const int idx = base + threadIdx.x;
    const int m = idx / (nc * 64), oct = idx - m * (nc * 64);
    const bool live = idx < cells;
    bool in;
    const u4_t *src = x_cell<MTS>(p, idx, c0, nc, in);
    u4_t v;
    if (PRE && base < XFirst<false>::kCells * kThreads) v = first.v[base / kThreads];
    else v = *src;
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
    if (t0 + r >= p.tiles) continue;
    const TileRef tr = tile_ref(p.ms, t0 + r);
#pragma unroll
    for (int e = 0; e < E; ++e) {
      const int m = 4 * q + e;
      if (m < p.M) store_y(tr, j, m, yacc[r][e] * mul, p.y_f16);
    }
  }
}

// fp8 x fp4 path, one unit (R tiles x 4 groups).  Lane 16qa + r reads A row
// r (token r / NPC, piece r % NPC) of each group.
template <int FMT, int MP, int NPC, int R, int E>
__device__ __forceinline__ void compute_fp4(const GemvParams &p, const char *lds, const Unit<FMT, R> &u, int c_local,
                                            float (&yacc)[R][4]) {
  const int lane = threadIdx.x & 63, qa = lane >> 4, r = lane & 15;
  // Lanes of A rows past NPC MP read row 0 again: an A row only feeds the
  // same row of the product, and those rows are never stored.
  const int rr = r < NPC * MP ? r : 0;
  const char *xa = lds + p.off_x + (c_local * 4 * NPC * MP + rr) * kRowBytes + qa * 32;
  const uint8_t *sa = reinterpret_cast<const uint8_t *>(lds + p.off_corr) + (c_local * 4 * MP + rr / NPC) * 4 + qa;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    const u4_t a0 = *reinterpret_cast<const u4_t *>(xa + g * NPC * MP * kRowBytes);
    const u4_t a1 = *reinterpret_cast<const u4_t *>(xa + g * NPC * MP * kRowBytes + 16);
    const int sc = sa[g * MP * 4];
#pragma unroll
    for (int r2 = 0; r2 < R; ++r2) {
      u4_t b;
      if constexpr (FMT == 1) b = q1_fp4(u.w[r2][g]);
      else b = tq2_fp4(u.w[r2][2 * g], u.w[r2][2 * g + 1]);
      const f4_t d = mfma_f8f4(a0, a1, b, sc);
      const float s = half_to_float(uint16_t(u.s[r2][g >> 1] >> (16 * (g & 1))));
#pragma unroll
      for (int e = 0; e < E; ++e) yacc[r2][e] = fmaf(s, d[e], yacc[r2][e]);
    }
  }
}

// Accumulator element e of lane 16qa + j is A row 4qa + e: with two pieces
// token 2qa + e / 2, piece e % 2; with three (one token) token 0, piece e,
// all in lane quarter 0.
template <int FMT, int NPC, int R, int E>
__device__ __forceinline__ void store_fp4(const GemvParams &p, int t0, const float (&yacc)[R][4]) {
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, qa = lane >> 4;
  const float mul = FMT == 1 ? 1.f : 0.5f;
#pragma unroll
  for (int r = 0; r < R; ++r) {
    if (t0 + r >= p.tiles) continue;
    const TileRef tr = tile_ref(p.ms, t0 + r);
    if constexpr (NPC == 3) {
      if (qa == 0) store_y(tr, j, 0, ((yacc[r][0] + yacc[r][1]) + yacc[r][2]) * mul, p.y_f16);
    } else {
#pragma unroll
      for (int tt = 0; tt < E / 2; ++tt) {
        const int m = 2 * qa + tt;
        if (m < p.M) store_y(tr, j, m, (yacc[r][2 * tt] + yacc[r][2 * tt + 1]) * mul, p.y_f16);
      }
    }
  }
}

// Position of a wave in its flat sequence of units: tile set iteration it,
// stage st, slot kl inside the stage.  Advanced incrementally (no divisions).
struct Cursor {
  int it, st, kl;
};

// Returns true when the cursor moved to the next tile set.
__device__ __forceinline__ bool advance(Cursor &c, int U, int n_stages) {
  if (++c.kl == U) {
    c.kl = 0;
    if (++c.st == n_stages) {
      c.st = 0;
      ++c.it;
      return true;
    }
  }
  return false;
}

// Waves per SIMD the kernel is built for (the second launch bound).  Four
// (two workgroups per CU) leave 128 registers per lane, which the fp8 x fp4
// path with four row tiles per wave and several tokens exceeds: it spilled
// 36-40 bytes per lane to scratch.  That variant is built for two waves per
// SIMD (one workgroup per CU), and the plan reads the residency it gets.
template <int MT, int R, bool FP4>
constexpr int gemv_min_waves() {
  return (FP4 && MT > 1 && R >= 4) ? 2 : 4;
}

// Each wave walks a flat sequence of units (tile set, chunk) with a ring of
// D units in flight: the loads of unit i + D - 1 are issued before unit i is
// computed, across chunk, stage and tile-set boundaries.
// FP4 selects the fp8 x fp4 path (MT = token slots MP, at most 8).  FULL:
// every matrix has whole row tiles and K whole chunks; the loads then take
// tile addresses resolved once per tile set and step a fixed stride per
// chunk (the general path resolves the tile and its ragged shape per unit).
template <int FMT, bool BF, int MT, int R, int D, bool FP4, bool FULL>
__global__ void __launch_bounds__(kThreads, (gemv_min_waves<MT, R, FP4>())) gemv_kernel(GemvParams p) {
  // Accumulator elements that can hold a token (fp4: A rows, two per token).
  // fp8 pieces per token: two for bf16 x, three for fp16 x (one token only).
  constexpr int NPC = BF ? 2 : 3;
  static_assert(!FP4 || BF || MT == 1, "fp16 x on the fp8 x fp4 path covers one token");
  constexpr int E = FP4 ? (MT == 1 ? NPC : 4) : (MT == 1 ? 1 : 4);
  constexpr int MTS = MT;                // token slots per x cell
  extern __shared__ __align__(16) char lds[];
  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;
  if constexpr (!FP4 && MTS < 16) {
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

  // The load side: its cursor, the tile set it reads (FULL) and one unit's
  // loads.  Units outside the sequence re-read chunk 0 of the current set.
  Cursor ld = {0, 0, 0};
  TileSet<R> lts;
  if constexpr (FULL) resolve_tiles<FMT, R>(p, lts, uni(tile0(ld)));
  auto load = [&](Unit<FMT, R> &u, bool in_seq) {
    const bool v = in_seq && is_valid(ld);
    if constexpr (FULL) load_full<FMT, R>(lts, u, uni(v ? chunk(ld) : 0));
    else load_unit<FMT, R>(p, u, uni(tile0(ld)), uni(chunk(ld)), v);
    if (advance(ld, U, p.n_stages)) {
      if constexpr (FULL) resolve_tiles<FMT, R>(p, lts, uni(tile0(ld)));
    }
  };

  // x of the whole K (when it fits): the thread's first item is loaded, then
  // the first D - 1 units' weights, then x is converted and staged.
  float yacc[R][4];
  Unit<FMT, R> ring[D];
  XFirst<FP4> xf;
  if (!restage) {
    if constexpr (FP4) fp4_item_load<MT>(p, threadIdx.x, 0, p.chunks, xf.v);
    else {
#pragma unroll
      for (int i = 0; i < XFirst<false>::kCells; ++i) {
        bool in;
        xf.v[i] = *x_cell<MTS>(p, threadIdx.x + i * kThreads, 0, p.chunks, in);
      }
    }
  }
#pragma unroll
  for (int d = 0; d < D - 1; ++d) load(ring[d], d < total);
  if (!restage) {
    if constexpr (FP4) stage_fp4<FMT, BF, MT, true>(p, lds, 0, p.chunks, xf);
    else stage_x<FMT, BF, MTS, true>(p, lds, 0, p.chunks, xf);
    lds_barrier();
  }

  Cursor cu = {0, 0, 0};
  for (int i0 = 0; i0 < total; i0 += D) {
#pragma unroll
    for (int d = 0; d < D; ++d) {
      const int i = i0 + d;
      // Every step issues its loads and no step leaves the loop early: each
      // path through the body then issues the same loads, so the wait before
      // a unit's MFMAs covers that unit only (wait counts are in issue order,
      // and the compiler keeps the fewest loads in flight that any path to
      // the wait leaves).
      load(ring[(d + D - 1) % D], i + D - 1 < total);
      if (i >= total) continue;

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
        lds_barrier();
        const int c0 = cu.st * p.SC;
        if constexpr (FP4) stage_fp4<FMT, BF, MT, false>(p, lds, c0, min(p.SC, p.chunks - c0), xf);
        else stage_x<FMT, BF, MTS, false>(p, lds, c0, min(p.SC, p.chunks - c0), xf);
        lds_barrier();
      }
      if (is_valid(cu)) {
        const int c_local = s + cu.kl * S;
        if constexpr (FP4) {
          compute_fp4<FMT, MT, NPC, R, E>(p, lds, ring[d], c_local, yacc);
        } else {
          const int xbase = xact ? p.off_x + (c_local * 64 * MTS + q * MTS + j) * 16 : 0;
          compute_unit<FMT, BF, R, E, MTS>(p, lds, ring[d], c_local, xbase, yacc);
        }
      }
      if (k_last) {
        const bool ts_ok = t0 < p.tiles;
        if (S == 1) {
          if (ts_ok) {
            if constexpr (FP4) store_fp4<FMT, NPC, R, E>(p, t0, yacc);
            else store_tiles<FMT, R, E>(p, t0, yacc);
          }
        } else {
          float *red = reinterpret_cast<float *>(lds + p.off_red);
#pragma unroll
          for (int r = 0; r < R; ++r)
#pragma unroll
            for (int e = 0; e < E; ++e) red[((wave * R + r) * E + e) * 64 + lane] = yacc[r][e];
          lds_barrier();
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
            if constexpr (FP4) store_fp4<FMT, NPC, R, E>(p, t0, tot);
            else store_tiles<FMT, R, E>(p, t0, tot);
          }
          lds_barrier();
        }
      }
      advance(cu, U, p.n_stages);
    }
  }
}

// Host-side choice of (R, S, grid), from timings of the decode shapes at one
// token on MI355X: a workgroup costs a fixed part (x staging) worth about two
// units plus its waves' units (one more per tile set when waves split K),
// and a CU that holds n workgroups runs each about 1 + 0.45 (n - 1) times
// slower.  So every (S, grid cap of 1, 2, ... workgroups per CU) is costed
// as (units per wave + 2) x that factor, and the cheapest wins.  The fp8
// split of x grows with K, so on that path the fixed part counts two units
// per 5120 of K: on the 5120 x 17408 down projection two row tiles per wave
// on 160 workgroups then win over one tile on 320 (8.35 against 8.8 us;
// with exact operands the one-tile plan stays ahead, 11.3 against 11.7).
template <int FMT, bool BF, int MT, int R, int D, bool FP4, bool FULL>
double make_plan(const LaunchArgs &a, GemvParams &p, int &grid, int &lds_bytes) {
  constexpr int NPC = BF ? 2 : 3;
  constexpr int E = FP4 ? (MT == 1 ? NPC : 4) : (MT == 1 ? 1 : 4);
  p = GemvParams{};
  const int64_t G = a.K / kGroup;
  p.ms = mat_set(a);
  p.X = a.X;
  p.M = int(a.M); p.K = int(a.K); p.G = int(G);
  p.tiles = int((a.N + 15) / 16);
  p.chunks = int((G + 3) / 4);
  p.tilesets = (p.tiles + R - 1) / R;
  p.y_f16 = a.y_f16;
  const int cus = num_cus();
  const void *kern = reinterpret_cast<const void *>(&gemv_kernel<FMT, BF, MT, R, D, FP4, FULL>);
  auto map = [&](int S, int SC) { return FP4 ? lds_map_fp4(MT, NPC, S, SC, R, E) : lds_map(MT, S, SC, R, E); };
  // x bytes a stage of SC chunks occupies.
  auto xbytes = [&](int SC) { return FP4 ? SC * 4 * (NPC * MT * kRowBytes + 4 * MT) : MT * SC * 1024; };

  double best = 1e300;
  GemvParams bp = p;
  int bgrid = 1, blds = 0;
  for (int S = 1; S <= 8; S *= 2) {
    if (S > 1 && S > p.chunks) break;
    GemvParams q = p;
    // Stage all chunks when the LDS map fits in 64 KB, else stream stages of
    // as many chunks as fit in 32 KB of x.
    int SC = (p.chunks + S - 1) / S * S;
    if (map(S, SC).total > 64 * 1024) {
      if (xbytes(S) > 32 * 1024) continue;
      SC = S;
      while (SC + S <= p.chunks && xbytes(SC + S) <= 32 * 1024) SC += S;
    }
    q.S = S;
    q.SC = SC;
    q.n_stages = (p.chunks + SC - 1) / SC;
    const LdsMap m = map(S, SC);
    q.off_corr = m.corr; q.off_x = m.x; q.off_red = m.red;
    const int P = kWaves / S;
    const int per_cu = resident_blocks(kern, kThreads, m.total);
    const int want = (q.tilesets + P - 1) / P;
    for (int n = 1; n <= per_cu; ++n) {
      const int g = max(1, min(want, cus * n));
      const int64_t rows = (int64_t)g * P;
      const int64_t its = (q.tilesets + rows - 1) / rows;
      // Waves that split K add their sums through LDS once per tile set
      // (two barriers): about one unit each.
      const double units = double(its) * R * ((p.chunks + S - 1) / S) + (S > 1 ? double(its) : 0.0);
      const int share = (g + cus - 1) / cus;
      const double fixed = FP4 && p.K > 5120 ? 2.0 * p.K / 5120.0 : 2.0;
      const double cost = (units + fixed) * (1.0 + 0.45 * (share - 1));
      if (cost < best) {
        best = cost;
        bp = q;
        bgrid = g;
        blds = m.total;
      }
      if (g == want) break;
    }
  }
  p = bp;
  grid = bgrid;
  lds_bytes = blds;
  return best;
}

template <int FMT, bool BF, int MT, bool FP4, int RA, int RB, bool FULL>
hipError_t launch_mt_full(const LaunchArgs &a) {
  GemvParams p1, p2;
  int g1, g2, l1, l2;
  // Ring depth: three units in flight for q1 (1 KB per tile each), two for
  // tq2 (2 KB per tile each) and for four-tile units, so that four waves per
  // SIMD fit in registers.
  constexpr int DA = (FMT == 1 && RA < 4) ? 3 : 2;
  constexpr int DB = (FMT == 1 && RB < 4) ? 3 : 2;
  const double c1 = make_plan<FMT, BF, MT, RA, DA, FP4, FULL>(a, p1, g1, l1);
  const double c2 = make_plan<FMT, BF, MT, RB, DB, FP4, FULL>(a, p2, g2, l2);
  if (a.plan) {
    const bool one = c1 < c2;
    const GemvParams &p = one ? p1 : p2;
    lowbit_plan &o = plan_record(a, LOWBIT_KERNEL_GEMV_STAGED, one ? g1 : g2, kThreads, one ? l1 : l2);
    o.token_slots = MT;
    o.operands = FP4 ? (BF ? LOWBIT_OPERANDS_FP8_FP4 : LOWBIT_OPERANDS_FP8X3_FP4)
                     : (BF ? LOWBIT_OPERANDS_BF16 : LOWBIT_OPERANDS_F16);
    o.whole_tiles = FULL;
    o.tiles_per_wave = one ? RA : RB;
    o.ring = one ? DA : DB;
    o.waves_per_tile = p.S;
    o.groups_per_range = 4 * ((p.chunks + p.S - 1) / p.S);
    o.groups_per_pass = 4 * p.SC;
    o.lds_offsets[0] = p.off_corr;
    o.lds_offsets[1] = p.off_x;
    o.lds_offsets[2] = p.off_red;
    return hipSuccess;
  }
  if (c1 < c2)
    hipLaunchKernelGGL((gemv_kernel<FMT, BF, MT, RA, DA, FP4, FULL>), dim3(g1), dim3(kThreads), l1, a.stream, p1);
  else
    hipLaunchKernelGGL((gemv_kernel<FMT, BF, MT, RB, DB, FP4, FULL>), dim3(g2), dim3(kThreads), l2, a.stream, p2);
  return hipGetLastError();
}

// Every matrix of the launch has whole row tiles and K whole chunks.
inline bool full_units(const LaunchArgs &a) {
  if (a.K % 512 != 0) return false;
  for (int i = 0; i < a.nmat; ++i)
    if (a.Ns[i] % 16 != 0) return false;
  return true;
}

template <int FMT, bool BF, int MT, bool FP4, int RA, int RB>
hipError_t launch_mt(const LaunchArgs &a) {
  return full_units(a) ? launch_mt_full<FMT, BF, MT, FP4, RA, RB, true>(a)
                       : launch_mt_full<FMT, BF, MT, FP4, RA, RB, false>(a);
}

// Path choice, from timings of the decode shapes on MI355X (the split
// kernel can run without a workspace only when it need not cut K, which its
// plan ensures for 65536 rows and more).
// Binary weights with bf16 x (fp8 x fp4 kernels):
//  * one token: the workgroup-staged kernel above (x of the whole K in LDS);
//  * 2..8 tokens: the staged kernel, or the 2-D split (row blocks x K
//    ranges, x converted once per block, gemv_split.hip) on long rows, on
//    2 tokens from 24576 rows, on 3+ tokens below 65536 rows (at 3-4
//    tokens only where the split's plan fills two thirds of the CUs),
//    and on 5+ tokens of very tall matrices;
//  * 9..16 tokens: waves that split K over three or more row tiles per
//    workgroup (gemv_kslice.hip) when K is 4..10 whole chunks and the matrix
//    has the tiles for it; else the 2-D split; without a workspace on a
//    small matrix, x loaded straight into registers (gemv_wide.hip).
// Binary weights with fp16 x at one token: the staged kernel on the fp8 x
// fp4 instruction with three pieces per value (fp16 has 11 significant bits).
// Exact f16 / bf16 operands (ternary weights, fp16 x): the staged kernel for
// up to 4 tokens unless the rows are long or the matrix tall, the 2-D split
// for 5..8 tokens on 8192+ rows or long rows and for 9..16 tokens (the
// K-sliced kernel first, as above), else the register kernel.
//
// The fp8 x fp4 kernels (the staged one with FP4, and the split) hold each
// 32-value activation block at one shared exponent: values within 2^7 of
// the block's largest stay exact (bf16 x, two pieces; fp16 x, three pieces:
// within 2^6), smaller ones carry an error below 2^-17 of it.  With binary weights every product of the block counts in the error
// bound (|w| = s throughout a group), so that error stays below 2^-12 of the
// bound's sum; a ternary zero can drop the large value from the sum, so tq2
// always takes exact operands.
// Whether the split kernel's plan for this call keeps at least two thirds
// of the CUs busy (asked of its own planner, which launches nothing when it
// records a plan).  At 4 tokens a matrix of 1088 row tiles gets 136 row
// blocks and no K cut from it, and there the staged kernel takes 9.9 us
// against 12.0 us; 182 blocks (2176 tiles, 12 waves each) tie with it at
// 4 tokens and win at 2 (11.9 against 12.3 us).
inline bool split_fills_chip(const LaunchArgs &a) {
  lowbit_plan pl{};
  LaunchArgs b = a;
  b.plan = &pl;
  if (launch_gemv_split(b) != hipSuccess) return false;
  return 3 * int64_t(pl.grid) >= 2 * int64_t(num_cus());
}

template <int FMT, bool BF>
hipError_t launch_fmt(const LaunchArgs &a) {
  const bool ws_ok = a.ws && a.ws_bytes >= gemv_split_workspace_bytes(a.M, a.N, a.K);
  const bool split_ok = ws_ok || a.N >= 65536;
  if constexpr (BF && FMT == 1) {
    constexpr int RB = 4;
    if (a.M > 8) {
      hipError_t e;
      if (launch_gemv_kslice(a, e)) return e;
      return split_ok ? launch_gemv_split(a) : launch_gemv_wide(a);
    }
    bool split = a.M >= 2 && ((ws_ok && (a.K >= 8192 || (a.M >= 3 ? a.N < 65536 : a.N >= 24576))) ||
                              (a.M > 4 && a.N >= 65536));
    if (split && a.M <= 4 && a.K < 8192) split = split_fills_chip(a);
    if (split) return launch_gemv_split(a);
    if (a.M <= 1) return launch_mt<FMT, BF, 1, true, 1, 2>(a);
    if (a.M <= 2) return launch_mt<FMT, BF, 2, true, 2, RB>(a);
    if (a.M <= 4) return launch_mt<FMT, BF, 4, true, 2, RB>(a);
    return launch_mt<FMT, BF, 8, true, 2, RB>(a);
  } else {
    if (a.M > 8) {
      hipError_t e;
      if (launch_gemv_kslice(a, e)) return e;
      return split_ok ? launch_gemv_split(a) : launch_gemv_wide(a);
    }
    if (a.M >= 2) {
      const bool split = a.K >= 8192 || (a.M > 4 ? a.N >= 8192 : (a.N >= 24576 && a.N < 65536));
      if (split && split_ok) return launch_gemv_split(a);
    }
    if (a.M <= 1) {
      // Binary weights, fp16 x, one token: three fp8 pieces per value on the
      // fp8 x fp4 instruction (one MFMA per tile and group, as for bf16 x).
      if constexpr (FMT == 1 && !BF) return launch_mt<FMT, BF, 1, true, 1, 2>(a);
      else return launch_mt<FMT, BF, 1, false, 1, 2>(a);
    }
    if (a.M <= 4) return launch_mt<FMT, BF, 4, false, 1, 2>(a);
    return launch_gemv_wide(a);
  }
}

}  // namespace

int64_t gemv_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  return fmt == 3 ? 0 : gemv_split_workspace_bytes(M, N, K);
}

hipError_t launch_gemv(const LaunchArgs &a) {
  // Token blocks of at most 16 rows share one pass over the weights.  A plan
  // query records the first block's launch and counts the blocks.
  for (int64_t m0 = 0; m0 < a.M; m0 += a.plan ? a.M : 16) {
    LaunchArgs b = a;
    b.M = a.M - m0 < 16 ? a.M - m0 : 16;
    b.X = a.X + m0 * a.K;
    for (int i = 0; i < a.nmat; ++i) b.Ys[i] = static_cast<char *>(a.Ys[i]) + m0 * a.Ns[i] * (a.y_f16 ? 2 : 4);
    b.Y = b.Ys[0];
    hipError_t e;
    if (a.fmt == 1) e = a.x_bf16 ? launch_fmt<1, true>(b) : launch_fmt<1, false>(b);
    else if (a.fmt == 2) e = a.x_bf16 ? launch_fmt<2, true>(b) : launch_fmt<2, false>(b);
    else e = launch_gemv_tq5(b);
    if (e != hipSuccess) return e;
    if (a.plan) a.plan->launches = int((a.M + 15) / 16);
  }
  return hipSuccess;
}

}  // namespace lowbit
