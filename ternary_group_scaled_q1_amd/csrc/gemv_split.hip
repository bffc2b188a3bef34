// Decode GEMV with a 2-D work split: Y[m][n] = sum_k X[m][k] t[n][k] s[n][k/128],
// up to 16 tokens.  Binary weights with bf16 x run on the fp8 x fp4 matrix
// instructions (below); ternary weights and fp16 x take exact f16 / bf16
// operands on v_mfma_f32_16x16x32 with x staged in LDS as it is (the same
// work split).
//
// A workgroup owns a row block (8 or 12 waves x R row tiles of 16 rows) and one
// K range of the matrix.  It converts the x of its K range once into LDS as
// exact fp8 pieces with per-32 E8M0 scales (split_x_quarter in device.hpp),
// in passes of GP groups that are double buffered: while the waves multiply
// pass p, the raw bf16 x of pass p + 1 is already in registers and is
// converted into the other buffer.  Every x value staged is then used by the
// 8R row tiles of the block, so the activations cross the L2 once per block
// instead of once per tile (16 tokens of x are as large as the weights that
// use them).
//
// Small matrices have too few row blocks to fill the chip, so their K is cut
// into KS ranges handled by different workgroups.  Each writes its fp32
// partial sums to the caller's workspace and increments the block's arrival
// counter; the last of the KS workgroups adds the KS partials in range
// order, which makes the result independent of which finished last, writes
// Y and resets the counter to 0.  The XCDs' L2 caches are not coherent with
// each other, and an agent-scope fence would write back and invalidate a
// whole L2 per workgroup, so the partials instead travel as agent-scope
// atomic stores and loads (emitted with the sc1 bit: they go to and come
// from the device's coherence point); each thread waits for its stores to
// complete and the workgroup synchronises before one thread increments the
// counter, and the last workgroup reads only after it saw the count.
//
// Per (row tile, group) the weights decode to fp4 (q1: +-1, tq2: 2t) with a
// shift and one bitwise op per 8 weights; up to 8 tokens one scaled
// 16x16x128 MFMA takes x as A rows (token, piece), at 16 tokens two chained
// MFMAs take the hi and then the lo pieces of all 16 tokens; the group's FP16
// scale is applied to the fresh fp32 tile (exact products), as on the
// aberweb.com page, section 4.1: the signs are decoded inside the kernel and
// no dense weight tensor exists.
#include <type_traits>

#include "device.hpp"
#include "gemv_common.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

// Waves per workgroup: 8, or 12 for launches whose row tiles exceed 8 per CU
// but not 12 (three tiles per SIMD instead of four at two tiles per wave).
constexpr int kSWaves = 8;

struct SplitParams {
  MatSet ms;           // the matrices (row tiles numbered across them)
  const uint16_t *X;   // [M][K]
  float *part;         // [KS][M][NV] partial sums (KS > 1)
  unsigned *count;     // [row_blocks] arrival counters, 0 between calls
  int M, K, G, tiles;
  int NV;          // launch rows: 16 x tiles
  int GK;          // groups per K range (a multiple of 4 when KS > 1)
  int KS;          // K ranges
  int GP;          // groups per staging pass (a multiple of 4)
  int row_blocks;  // ceil(tiles / (NW R))
  int y_f16;
  int buf_bytes;   // LDS bytes of one staging buffer
};

// Operand modes: kFp4 (bf16 x as fp8 pieces, binary weights as fp4, scaled
// 16x16x128 MFMA) or exact f16 / bf16 operands on v_mfma_f32_16x16x32
// (kBf16, kF16: x staged as it is, weights decoded to exact +-1 / 2t).
constexpr int kFp4 = 0, kBf16 = 1, kF16 = 2;

// LDS of one staging buffer.  kFp4: GP groups x 2*MP A rows, then GP*MP*4
// scale bytes.  Exact modes: 16-byte cells (group, k-step u, quarter q,
// token m) of x[m][128 g + 32 u + 8 q .. + 8], then one zero cell.
__host__ __device__ constexpr int split_buf_bytes(int MP, int GP, int MODE) {
  return MODE == kFp4 ? (GP * 2 * MP * kRowBytes + GP * MP * 4 + 15) / 16 * 16 : GP * 16 * MP * 16 + 16;
}

// Raw x of one (token, group, lane quarter) item, held between its load and
// its conversion.
struct RawQ {
  u4_t v[4];  // as loaded: zeroed only when converted, so the load waits nowhere
  bool in;    // the item holds x (a token below M, a group of the pass)
};

// Token slot m, lane quarter q and pass group gl of an item.  Exact modes
// number the items token slot fastest, so the 16-byte LDS writes of
// neighbouring lanes go to neighbouring cells; numbered lane quarter
// fastest, all lanes of one token hit the same banks (the group stride is a
// multiple of the bank width), 6 conflicts per LDS instruction on the
// ternary launches.  The fp8-piece path keeps lane quarter fastest: token
// slot fastest was 3-5% slower there (its rows are 144 bytes apart, so it
// conflicts little either way).
template <int MP, int MODE>
__device__ __forceinline__ void item_coords(int item, int GP, int &m, int &q, int &gl) {
  if constexpr (MODE == kFp4) {
    q = item & 3;
    const int rest = item >> 2;
    gl = rest % GP;
    m = rest / GP;
  } else {
    m = item % MP;
    const int rest = item / MP;
    q = rest & 3;
    gl = rest >> 2;
  }
}

template <int MP, int MODE>
__device__ __forceinline__ void load_raw(const SplitParams &p, RawQ &r, int g0, int np_groups, int item, bool &live) {
  int m, q, gl;
  item_coords<MP, MODE>(item, p.GP, m, q, gl);
  live = item < MP * p.GP * 4;
  r.in = live && m < p.M && gl < np_groups;
  const uint16_t *src = p.X + (r.in ? (int64_t)m * p.K + 128 * (g0 + gl) + 8 * q : 0);
#pragma unroll
  for (int u = 0; u < 4; ++u) r.v[u] = *reinterpret_cast<const u4_t *>(src + 32 * u);
}

template <int FMT, int MP, int MODE>
__device__ __forceinline__ void convert_raw(const SplitParams &p, const RawQ &r, char *buf, int item) {
  int m, q, gl;
  item_coords<MP, MODE>(item, p.GP, m, q, gl);
  const u4_t z = {0u, 0u, 0u, 0u};
  u4_t v[4];
#pragma unroll
  for (int u = 0; u < 4; ++u) v[u] = r.in ? r.v[u] : z;
  if constexpr (MODE != kFp4) {
#pragma unroll
    for (int u = 0; u < 4; ++u) *reinterpret_cast<u4_t *>(buf + (((gl * 4 + u) * 4 + q) * MP + m) * 16) = v[u];
    return;
  }
  XQuarter xq;
  split_x_regs<FMT>(v, xq);
  // A rows of group gl: (token, piece) pairs 2m + piece up to 8 tokens; at 16
  // tokens the hi pieces of all tokens, then the lo pieces.
  char *row = buf + (gl * 2 * MP + (MP > 8 ? m : 2 * m)) * kRowBytes;
  char *lrow = row + (MP > 8 ? MP : 1) * kRowBytes;
  const int qa = 2 * (q & 1), half = 16 * (q >> 1);
  *reinterpret_cast<u4_t *>(row + qa * 32 + half) = xq.h0;
  *reinterpret_cast<u4_t *>(row + (qa + 1) * 32 + half) = xq.h1;
  *reinterpret_cast<u4_t *>(lrow + qa * 32 + half) = xq.l0;
  *reinterpret_cast<u4_t *>(lrow + (qa + 1) * 32 + half) = xq.l1;
  reinterpret_cast<uint8_t *>(buf + p.GP * 2 * MP * kRowBytes)[(gl * MP + m) * 4 + q] = xq.sb;
}

// One chunk (4 groups at buffer group offset gb) for R tiles, up to 8 tokens:
// lane 16qa + r reads A row r (token r / 2, piece r % 2), so one MFMA per
// (tile, group) covers both pieces.
template <int FMT, int MP, int R>
__device__ __forceinline__ void compute_chunk(const SplitParams &p, const char *buf, const Unit<FMT, R> &u, int gb,
                                              int ng, float (&yacc)[R][1][4]) {
  const int lane = threadIdx.x & 63, qa = lane >> 4, r = lane & 15;
  const bool arow = r < 2 * MP;
  const int rr = arow ? r : 0;
  const u4_t z = {0u, 0u, 0u, 0u};
  const uint8_t *scb = reinterpret_cast<const uint8_t *>(buf + p.GP * 2 * MP * kRowBytes);
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    if (gi >= ng) break;  // wave-uniform: groups past K in the last chunk
    const int gl = gb + gi;
    const char *xa = buf + (gl * 2 * MP + rr) * kRowBytes + qa * 32;
    const u4_t v0 = *reinterpret_cast<const u4_t *>(xa);
    const u4_t v1 = *reinterpret_cast<const u4_t *>(xa + 16);
    const u4_t a0 = arow ? v0 : z;
    const u4_t a1 = arow ? v1 : z;
    const int sa = scb[(gl * MP + (rr >> 1)) * 4 + qa];
#pragma unroll
    for (int r2 = 0; r2 < R; ++r2) {
      u4_t b;
      if constexpr (FMT == 1) b = q1_fp4(u.w[r2][gi]);
      else b = tq2_fp4(u.w[r2][2 * gi], u.w[r2][2 * gi + 1]);
      const float s = half_to_float(uint16_t(u.s[r2][gi >> 1] >> (16 * (gi & 1))));
      const f4_t d = mfma_f8f4(a0, a1, b, sa);
#pragma unroll
      for (int e = 0; e < 4; ++e) yacc[r2][0][e] = fmaf(s, d[e], yacc[r2][0][e]);
    }
  }
}

// The same at 16 tokens: lane 16qa + r reads the hi-piece row of token r, then
// its lo-piece row; the two MFMAs of a (tile, group) share the weights and the
// x scales and chain into one fp32 tile (token 4qa + e in element e), so the
// group's FP16 scale takes one multiply-add per output instead of one per
// piece.
template <int FMT, int MP, int R>
__device__ __forceinline__ void compute_chunk16(const SplitParams &p, const char *buf, const Unit<FMT, R> &u, int gb,
                                                int ng, float (&yacc)[R][1][4]) {
  const int lane = threadIdx.x & 63, qa = lane >> 4, r = lane & 15;
  const uint8_t *scb = reinterpret_cast<const uint8_t *>(buf + p.GP * 2 * MP * kRowBytes);
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    if (gi >= ng) break;  // wave-uniform: groups past K in the last chunk
    const int gl = gb + gi;
    const char *xh = buf + (gl * 2 * MP + r) * kRowBytes + qa * 32;
    const char *xl = xh + MP * kRowBytes;
    const u4_t h0 = *reinterpret_cast<const u4_t *>(xh);
    const u4_t h1 = *reinterpret_cast<const u4_t *>(xh + 16);
    const u4_t l0 = *reinterpret_cast<const u4_t *>(xl);
    const u4_t l1 = *reinterpret_cast<const u4_t *>(xl + 16);
    const int sa = scb[(gl * MP + r) * 4 + qa];
#pragma unroll
    for (int r2 = 0; r2 < R; ++r2) {
      u4_t b;
      if constexpr (FMT == 1) b = q1_fp4(u.w[r2][gi]);
      else b = tq2_fp4(u.w[r2][2 * gi], u.w[r2][2 * gi + 1]);
      const float s = half_to_float(uint16_t(u.s[r2][gi >> 1] >> (16 * (gi & 1))));
      const f4_t d = mfma_f8f4_acc(l0, l1, b, sa, mfma_f8f4(h0, h1, b, sa));
#pragma unroll
      for (int e = 0; e < 4; ++e) yacc[r2][0][e] = fmaf(s, d[e], yacc[r2][0][e]);
    }
  }
}

// Exact modes: one chunk (4 groups at buffer group offset gb) for R tiles.
// Lane 16q + j reads the cell of token j (the zero cell for j >= MP); the
// group's 4 k-steps fill a fresh tile that is added as s * tile.
template <int FMT, int MP, int R, int MODE>
__device__ __forceinline__ void compute_chunk_ex(const SplitParams &p, const char *buf, const Unit<FMT, R> &u, int gb,
                                                 int ng, float (&yacc)[R][1][4]) {
  constexpr bool BF = MODE == kBf16;
  const int lane = threadIdx.x & 63, q = lane >> 4, j = lane & 15;
  const bool tok = j < MP;
  const int zero = p.GP * 16 * MP * 16;
#pragma unroll
  for (int gi = 0; gi < 4; ++gi) {
    if (gi >= ng) break;  // wave-uniform: groups past K in the last chunk
    const int gl = gb + gi;
    u4_t a[4];
#pragma unroll
    for (int uu = 0; uu < 4; ++uu)
      a[uu] = *reinterpret_cast<const u4_t *>(buf + (tok ? (((gl * 4 + uu) * 4 + q) * MP + j) * 16 : zero));
#pragma unroll
    for (int r2 = 0; r2 < R; ++r2) {
      f4_t acc;
#pragma unroll
      for (int uu = 0; uu < 4; ++uu) {
        u4_t b;
        if constexpr (FMT == 1) b = q1_operand_pm1<BF>(u.w[r2][gi], uu);
        else b = tq2_operand(u.w[r2][2 * gi + (uu >> 1)], uu);
        acc = uu == 0 ? mfma16x16x32_zero<BF>(a[uu], b) : mfma16x16x32<BF>(a[uu], b, acc);
      }
      const float s = half_to_float(uint16_t(u.s[r2][gi >> 1] >> (16 * (gi & 1))));
#pragma unroll
      for (int e = 0; e < 4; ++e) yacc[r2][0][e] = fmaf(s, acc[e], yacc[r2][0][e]);
    }
  }
}

// FULL: every matrix has whole row tiles and K whole chunks; a wave's tiles
// are fixed for the launch, so their addresses are resolved once and each
// chunk is one load per tile at a fixed stride (the general path resolves
// the tile and its ragged shape per chunk).
//
// CPP > 0: every staging pass is CPP chunks (a compile-time count; CPP is
// even, so a chunk's ring slot is fixed), the loop walks passes and the raw
// x of the next pass is loaded on every path (past the range as zeros from a
// clamped address).  Between the raw x of a pass and its conversion at the
// next pass boundary there are then exactly CPP units of weight loads on
// every path, so the wait for x is a count that leaves those in flight.  In
// the general loop (CPP = 0) the number of loads between the two differs
// between paths and the compiler waits for every load at each boundary,
// which drains the weight ring once per pass.
template <int FMT, int MP, int R, int MODE, bool FULL, int NW, int CPP>
__global__ void __launch_bounds__(64 * NW, NW <= 8 ? 2 : 1) gemv_split_kernel(SplitParams p) {
  constexpr int kThreads = 64 * NW;
  // One fp32 tile per row tile: fp4 A rows hold (token, piece) pairs for up
  // to 8 tokens, or at 16 tokens one token per row with the pieces chained;
  // exact operands hold 16 tokens per MFMA.
  extern __shared__ __align__(16) char lds[];
  __shared__ int last_flag;
  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;
  const int ks = blockIdx.x % p.KS, rb = blockIdx.x / p.KS;
  const int g0 = ks * p.GK;
  const int ng = uni(min(p.GK, p.G - g0));  // groups of this K range
  const int nchunks = (ng + 3) / 4;
  const int c0 = g0 / 4;
  const int t0 = uni(rb * NW * R + wave * R);
  const float mul = FMT == 1 ? 1.f : 0.5f;  // ternary operands carry 2t

  // x of pass 0 is loaded first, then the first two chunks of weights, so
  // that waiting for x (an in-order count) leaves the weights in flight.
  const int npass = (ng + p.GP - 1) / p.GP;
  const int cpp = p.GP / 4;  // chunks per pass
  RawQ raw;
  bool live;
  load_raw<MP, MODE>(p, raw, g0, min(p.GP, ng), threadIdx.x, live);

  // Weights: a ring of two units.  Every step computes one chunk and issues
  // the load of the chunk two ahead, clamped to the range's last chunk, so
  // that every path through the loop issues the same loads and the wait
  // before a chunk's MFMAs covers that chunk only.
  TileSet<R> ts;
  if constexpr (FULL) resolve_tiles<FMT, R>(p, ts, t0);
  auto load = [&](Unit<FMT, R> &u, int c) {
    if constexpr (FULL) load_full<FMT, R>(ts, u, c0 + c);
    else load_unit<FMT, R>(p, u, t0, c0 + c, true);
  };
  Unit<FMT, R> ring[2];
  load(ring[0], 0);
  load(ring[1], min(1, nchunks - 1));

  if (live) convert_raw<FMT, MP, MODE>(p, raw, lds, threadIdx.x);
  if constexpr (MODE != kFp4) {
    if (threadIdx.x == 0) {
      *reinterpret_cast<u4_t *>(lds + p.GP * 16 * MP * 16) = u4_t{0u, 0u, 0u, 0u};
      *reinterpret_cast<u4_t *>(lds + p.buf_bytes + p.GP * 16 * MP * 16) = u4_t{0u, 0u, 0u, 0u};
    }
  }
  lds_barrier();
  // The raw x of pass 1 goes out while pass 0 is multiplied.
  if (CPP > 0 || npass > 1) load_raw<MP, MODE>(p, raw, g0 + p.GP, min(p.GP, ng - p.GP), threadIdx.x, live);

  float yacc[R][1][4];
#pragma unroll
  for (int r = 0; r < R; ++r)
#pragma unroll
    for (int e = 0; e < 4; ++e) yacc[r][0][e] = 0.f;

  auto compute = [&](const char *cur, const Unit<FMT, R> &u, int cl, int png) {
    if constexpr (MODE == kFp4 && MP > 8) compute_chunk16<FMT, MP, R>(p, cur, u, 4 * cl, min(4, png - 4 * cl), yacc);
    else if constexpr (MODE == kFp4) compute_chunk<FMT, MP, R>(p, cur, u, 4 * cl, min(4, png - 4 * cl), yacc);
    else compute_chunk_ex<FMT, MP, R, MODE>(p, cur, u, 4 * cl, min(4, png - 4 * cl), yacc);
  };

  if constexpr (CPP > 0) {
    for (int ps = 0; ps < npass; ++ps) {
      if (ps > 0) {
        // The x of pass ps, loaded during pass ps - 1, goes into the buffer
        // of pass ps - 2 (every wave left that pass before the previous
        // barrier); then the raw x of pass ps + 1 goes out.
        if (live) convert_raw<FMT, MP, MODE>(p, raw, lds + (ps & 1) * p.buf_bytes, threadIdx.x);
        lds_barrier();
        const int nx = (ps + 1) * p.GP;
        load_raw<MP, MODE>(p, raw, g0 + nx, min(p.GP, ng - nx), threadIdx.x, live);
      }
      const char *cur = lds + (ps & 1) * p.buf_bytes;
      const int png = min(p.GP, ng - ps * p.GP);
#pragma unroll
      for (int cl = 0; cl < CPP; ++cl) {
        const int cc = ps * CPP + cl;  // chunk inside the K range
        if (cc < nchunks) compute(cur, ring[cl % 2], cl, png);
        load(ring[cl % 2], min(cc + 2, nchunks - 1));
      }
    }
  } else {
  for (int c = 0; c < nchunks; c += 2) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int cc = c + h;  // chunk inside the K range
      if (cc < nchunks) {
        const int ps = cc / cpp, cl = cc - ps * cpp;
        if (ps > 0 && cl == 0) {
          // First chunk of pass ps: its x, loaded during pass ps - 1, goes into
          // the buffer of pass ps - 2 (every wave left that pass before the
          // previous barrier); then the raw x of pass ps + 1 goes out.
          if (live) convert_raw<FMT, MP, MODE>(p, raw, lds + (ps & 1) * p.buf_bytes, threadIdx.x);
          lds_barrier();
          const int nx = (ps + 1) * p.GP;
          if (ps + 1 < npass) load_raw<MP, MODE>(p, raw, g0 + nx, min(p.GP, ng - nx), threadIdx.x, live);
        }
        const char *cur = lds + (ps & 1) * p.buf_bytes;
        const int png = min(p.GP, ng - ps * p.GP);
        compute(cur, ring[h], cl, png);
      }
      load(ring[h], min(cc + 2, nchunks - 1));
    }
  }
  }

  // This lane's outputs: (tile r, token m, value).  fp4 up to 8 tokens:
  // element e of lane 16qa + j is A row 4qa + e (token 2 qa + e / 2, piece
  // e % 2; the pieces add here); fp4 at 16 tokens and exact: token 4q + e.
  const int j = lane & 15, qa = lane >> 4;
  auto each_output = [&](auto f) {
#pragma unroll
    for (int r = 0; r < R; ++r) {
      if constexpr (MODE == kFp4 && MP <= 8) {
#pragma unroll
        for (int tt = 0; tt < 2; ++tt) f(r, 2 * qa + tt, yacc[r][0][2 * tt] + yacc[r][0][2 * tt + 1]);
      } else {
#pragma unroll
        for (int e = 0; e < 4; ++e) f(r, 4 * qa + e, yacc[r][0][e]);
      }
    }
  };
  if (p.KS == 1) {
    each_output([&](int r, int m, float v) {
      if (t0 + r < p.tiles && m < p.M) store_y(tile_ref(p.ms, t0 + r), j, m, v * mul, p.y_f16);
    });
    return;
  }

  // K split across workgroups: publish this range's partial sums (at launch
  // rows, every row of a tile included).
  // Memory ordering.  All three steps below are relaxed atomics, so the HIP
  // memory model alone orders nothing between them; the order comes from
  // gfx950's memory pipeline, as follows.
  //  * Agent-scope atomic stores and loads compile to global_store / load
  //    with sc1: they write through to, and read from, the device's
  //    coherence point, past this XCD's own L2, so no stale copy can be read
  //    and no dirty copy can stay behind in another XCD's L2.
  //  * s_waitcnt vmcnt(0) returns only once this thread's stores have been
  //    acknowledged, and the barrier holds thread 0 until every thread of
  //    the workgroup has passed its own wait.
  //  * The counter add is issued after that barrier.  Agent-scope atomics
  //    are coherent across the XCDs (one order of adds per counter).  The
  //    last workgroup issues its loads only after its add has returned:
  //    they depend on the result through the LDS flag and a barrier.
  // A release / acquire pair would add an L2 write-back before the add and
  // an L2 invalidate after it, on every workgroup of every launch.  The
  // partial sums never pass through an L2, so neither is needed.
  each_output([&](int r, int m, float v) {
    if (t0 + r < p.tiles && m < p.M)
      __hip_atomic_store(p.part + ((int64_t)ks * p.M + m) * p.NV + 16 * (t0 + r) + j, v, __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  });
  __builtin_amdgcn_s_waitcnt(0);  // this thread's partial stores have completed
  __syncthreads();
  if (threadIdx.x == 0)
    last_flag = __hip_atomic_fetch_add(p.count + rb, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                unsigned(p.KS - 1);
  __syncthreads();
  if (!last_flag) return;
  // Last workgroup of the block: Y = sum over ranges in range order.  The
  // partials come from the device's coherence point, so a thread issues the
  // loads of KR ranges for each of 4 outputs before it adds any of them
  // (addresses clamped, values past KS unused) instead of paying that latency
  // once per range; KR = 4 up to 4 ranges (no duplicate loads for the common
  // 2 or 3), else 8.
  const int n0 = rb * NW * R * 16;
  const int rows = min(NW * R * 16, p.NV - n0);
  const int outs = p.M * rows;
  constexpr int kOut = 4;
  auto reduce = [&](auto kr) {
    constexpr int KR = decltype(kr)::value;
    for (int base = 0; base < outs; base += kOut * kThreads) {
      int pm[kOut], pn[kOut];
      float v[kOut];
#pragma unroll
      for (int o = 0; o < kOut; ++o) {
        const int idx = min(base + o * kThreads + int(threadIdx.x), outs - 1);
        pm[o] = idx / rows;
        pn[o] = n0 + idx % rows;
        v[o] = 0.f;
      }
      for (int k0 = 0; k0 < p.KS; k0 += KR) {
        float pv[kOut][KR];
#pragma unroll
        for (int o = 0; o < kOut; ++o)
#pragma unroll
          for (int k = 0; k < KR; ++k)
            pv[o][k] = __hip_atomic_load(p.part + ((int64_t)min(k0 + k, p.KS - 1) * p.M + pm[o]) * p.NV + pn[o],
                                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
#pragma unroll
        for (int o = 0; o < kOut; ++o)
#pragma unroll
          for (int k = 0; k < KR; ++k)
            if (k0 + k < p.KS) v[o] += pv[o][k];
      }
#pragma unroll
      for (int o = 0; o < kOut; ++o)
        if (base + o * kThreads + int(threadIdx.x) < outs)
          store_y(tile_ref(p.ms, pn[o] >> 4), pn[o] & 15, pm[o], v[o] * mul, p.y_f16);
    }
  };
  if (p.KS <= 4) reduce(std::integral_constant<int, 4>{});
  else reduce(std::integral_constant<int, 8>{});
  if (threadIdx.x == 0) __hip_atomic_store(p.count + rb, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Largest pass (groups, a multiple of 4) whose x fits in one item per thread
// and whose two buffers fit in 80 KB of LDS (two workgroups per CU fit in
// the 160 KB of a gfx950 CU).
inline int pass_groups(int MP, int G, int MODE, int threads) {
  int gp = 4;
  while (gp + 4 <= 128 && MP * (gp + 4) * 4 <= threads && 2 * split_buf_bytes(MP, gp + 4, MODE) <= 80 * 1024) gp += 4;
  const int g4 = (G + 3) / 4 * 4;
  return gp < g4 ? gp : g4;
}

// Workspace: kMaxCounters arrival counters at offset 0 (a fixed place, so
// that calls of any shape sharing one workspace find them zero), then the
// partial sums.  K is cut into at most kMaxKS ranges, and only while the
// partials of all ranges stay within kMaxPartBytes (large matrices fill the
// chip with row blocks alone, and their partials would cost as much traffic
// as the weights) and the row blocks have counters.
constexpr int kMaxKS = 16;
constexpr int64_t kMaxPartBytes = 8 << 20;
constexpr int kMaxCounters = 8192;
constexpr int64_t kPartOffset = kMaxCounters * 4;

int64_t split_ws_bytes(int64_t M, int64_t N, int KS) {
  return KS <= 1 ? 0 : kPartOffset + (int64_t)KS * M * N * 4;
}

struct SplitPlan {
  SplitParams p;
  int grid = 0;
  int lds = 0;
};

// Parameters of the launch with R row tiles per wave and K cut into ranges
// of gk groups (false if the workspace, the partial-sum area or the counters
// cannot hold that cut).
template <int FMT, int MP, int R, int MODE, bool FULL, int NW>
bool make_split(const LaunchArgs &a, int gk, SplitPlan &pl) {
  SplitParams p{};
  p.ms = mat_set(a);
  p.X = a.X;
  p.M = int(a.M); p.K = int(a.K); p.G = int(a.K / kGroup);
  p.tiles = int((a.N + 15) / 16);
  p.NV = 16 * p.tiles;
  p.y_f16 = a.y_f16;
  p.row_blocks = (p.tiles + NW * R - 1) / (NW * R);
  p.GP = pass_groups(MP, p.G, MODE, 64 * NW);
  p.buf_bytes = split_buf_bytes(MP, p.GP, MODE);
  gk = gk < p.G ? gk : p.G;
  const int KS = (p.G + gk - 1) / gk;
  if (KS > kMaxKS) return false;
  if (KS > 1 && (gk % 4 || (int64_t)KS * a.M * p.NV * 4 > kMaxPartBytes || p.row_blocks > kMaxCounters ||
                 split_ws_bytes(a.M, p.NV, KS) > a.ws_bytes))
    return false;
  p.GK = gk;
  p.KS = KS;
  pl.p = p;
  pl.grid = p.row_blocks * KS;
  pl.lds = 2 * p.buf_bytes;
  return true;
}

template <int FMT, int MP, int MODE, bool FULL, int CPP>
hipError_t launch_split_plan(const LaunchArgs &a, const SplitPlan &pl, int NW, int R) {
  const dim3 grid(pl.grid), block(64 * NW);
  if (NW == 12)
    hipLaunchKernelGGL((gemv_split_kernel<FMT, MP, 1, MODE, FULL, 12, CPP>), grid, block, pl.lds, a.stream, pl.p);
  else if (R == 1)
    hipLaunchKernelGGL((gemv_split_kernel<FMT, MP, 1, MODE, FULL, kSWaves, CPP>), grid, block, pl.lds, a.stream, pl.p);
  else if (R == 2)
    hipLaunchKernelGGL((gemv_split_kernel<FMT, MP, 2, MODE, FULL, kSWaves, CPP>), grid, block, pl.lds, a.stream, pl.p);
  else
    hipLaunchKernelGGL((gemv_split_kernel<FMT, MP, 4, MODE, FULL, kSWaves, CPP>), grid, block, pl.lds, a.stream, pl.p);
  return hipGetLastError();
}

// Plan, from timings of the decode shapes at 2..16 tokens on MI355X: a CU
// that holds two workgroups runs each about 1.45x slower, and a workgroup's
// time is a fixed part (x staging, the K-range reduction, launch) plus a
// part per group of its K range.  So: the fewest row tiles per wave whose
// row blocks fit one per CU, then the most K ranges that keep the grid
// within the CUs (each range shortens every workgroup).  Between 8 and 12
// row tiles per CU a workgroup of 12 waves with one tile each keeps three
// tiles per SIMD where 8 waves of two tiles would hold four.  Matrices too
// tall for that take two tiles per wave and the whole of K (fewer rows per
// wave would only add waves that wait their turn; more hold too many
// registers).
template <int FMT, int MP, int MODE, bool FULL>
hipError_t launch_split_full(const LaunchArgs &a) {
  const int cus = num_cus();
  const int tiles = int((a.N + 15) / 16), G = int(a.K / kGroup);
  int NW = kSWaves, R = 1;
  if ((tiles + 7) / 8 <= cus) R = 1;
  else if ((tiles + 11) / 12 <= cus) NW = 12;
  else R = (tiles + 15) / 16 <= cus ? 2 : ((tiles + 31) / 32 <= cus ? 4 : 2);
  const int blocks = (tiles + NW * R - 1) / (NW * R);
  SplitPlan pl;
  auto make = [&](int gk) {
    if (NW == 12) return make_split<FMT, MP, 1, MODE, FULL, 12>(a, gk, pl);
    if (R == 1) return make_split<FMT, MP, 1, MODE, FULL, kSWaves>(a, gk, pl);
    if (R == 2) return make_split<FMT, MP, 2, MODE, FULL, kSWaves>(a, gk, pl);
    return make_split<FMT, MP, 4, MODE, FULL, kSWaves>(a, gk, pl);
  };
  bool ok = false;
  if (blocks <= cus) {
    // Most ranges first: gk = 4, 8, ... groups (a multiple of 4).
    for (int gk = 4; gk < G + 4 && !ok; gk += 4) {
      const int ks = (G + gk - 1) / gk;
      if ((int64_t)blocks * ks > cus && gk < G) continue;
      ok = make(gk);
    }
  } else {
    R = 2;
    ok = make(G);
  }
  if (!ok) return hipErrorInvalidValue;
  if (pl.p.KS > 1) {
    pl.p.count = static_cast<unsigned *>(a.ws);
    pl.p.part = reinterpret_cast<float *>(static_cast<char *>(a.ws) + kPartOffset);
  }
  if (a.plan) {
    lowbit_plan &o = plan_record(a, LOWBIT_KERNEL_GEMV_SPLIT, pl.grid, 64 * NW, pl.lds);
    o.token_slots = MP;
    o.operands = MODE == kFp4 ? LOWBIT_OPERANDS_FP8_FP4 : (MODE == kBf16 ? LOWBIT_OPERANDS_BF16 : LOWBIT_OPERANDS_F16);
    o.whole_tiles = FULL;
    o.tiles_per_wave = NW == 12 ? 1 : R;
    o.k_ranges = pl.p.KS;
    o.groups_per_range = pl.p.GK;
    o.groups_per_pass = pl.p.GP;
    o.ring = 2;
    return hipSuccess;
  }
  // Sixteen tokens stage x in passes of two chunks (pass_groups): those
  // launches take the pass-structured loop.
  if (MP == 16 && pl.p.GP == 8) return launch_split_plan<FMT, MP, MODE, FULL, 2>(a, pl, NW, R);
  return launch_split_plan<FMT, MP, MODE, FULL, 0>(a, pl, NW, R);
}

// Every matrix of the launch has whole row tiles and K whole chunks.
inline bool split_full(const LaunchArgs &a) {
  if (a.K % 512 != 0) return false;
  for (int i = 0; i < a.nmat; ++i)
    if (a.Ns[i] % 16 != 0) return false;
  return true;
}

template <int FMT, int MP, int MODE>
hipError_t launch_split_mp(const LaunchArgs &a) {
  return split_full(a) ? launch_split_full<FMT, MP, MODE, true>(a) : launch_split_full<FMT, MP, MODE, false>(a);
}

template <int FMT, int MODE>
hipError_t launch_split_fmt(const LaunchArgs &a) {
  if constexpr (MODE == kFp4) {
    if (a.M <= 1) return launch_split_mp<FMT, 1, MODE>(a);
    if (a.M <= 2) return launch_split_mp<FMT, 2, MODE>(a);
    if (a.M <= 4) return launch_split_mp<FMT, 4, MODE>(a);
    if (a.M <= 8) return launch_split_mp<FMT, 8, MODE>(a);
    return launch_split_mp<FMT, 16, MODE>(a);
  } else {
    // Exact operands take 16 token slots from two tokens on: the 16-slot
    // launches stage x in passes of two chunks on the pass-structured loop,
    // and with 4 slots (passes of eight chunks, the general loop) the
    // 27B-class tq2 GEMVs at 2-4 tokens took 19.1-19.3 us on 34816 x 5120
    // and 13.5-14.1 us on 5120 x 17408, against 16.2-16.6 and 12.5-13.0 us
    // with 16.  The fp8-piece path keeps its 2, 4 and 8 slots: there one
    // MFMA per (tile, group) covers both pieces of up to 8 tokens, and 16
    // slots were 10-30% slower.
    if (a.M <= 1) return launch_split_mp<FMT, 1, MODE>(a);
    return launch_split_mp<FMT, 16, MODE>(a);
  }
}

}  // namespace

int64_t gemv_split_workspace_bytes(int64_t M, int64_t N, int64_t K) {
  // The counters plus the largest partial-sum area any plan may use
  // (16-token launches).
  const int64_t m = M < 16 ? M : 16;
  N = (N + 15) / 16 * 16;  // partial sums are kept for whole row tiles
  int64_t ks = kMaxPartBytes / (m * N * 4);
  if (ks > kMaxKS) ks = kMaxKS;
  if (ks > K / kGroup) ks = K / kGroup;
  if (ks < 2 || ((N + 15) / 16 + 7) / 8 > kMaxCounters) return 0;
  return split_ws_bytes(m, N, int(ks));
}

hipError_t launch_gemv_split(const LaunchArgs &a) {
  // fp8 pieces of x only with binary weights (their error bound needs every
  // product of a block to count): tq2 and fp16 x take exact operands.
  if (a.fmt == 1) return a.x_bf16 ? launch_split_fmt<1, kFp4>(a) : launch_split_fmt<1, kF16>(a);
  return a.x_bf16 ? launch_split_fmt<2, kBf16>(a) : launch_split_fmt<2, kF16>(a);
}

}  // namespace lowbit
