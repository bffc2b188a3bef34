// Prefill GEMM  Y[m][n] = sum_k X[m][k] t[n][k] s[n][k/128]  for large M.
//
// Prompt processing is compute-bound (aberweb.com page, summary section 3),
// so this path is a dense contraction on the matrix cores: each wave decodes
// its own weight operands straight from the packed bits in registers into
// exact +-1 / 0 f16/bf16 halves and issues v_mfma_f32_16x16x32 against
// activation tiles staged in LDS.  The FP16 scale is applied once per group
// in fp32: each group accumulates into a fresh tile that is then added as
// s * tile (products exact, the scale is never rounded to bf16).
//
// Workgroup = 8 waves (two per SIMD, so one's MFMAs overlap the other's
// decode and waits) in 2 rows along M x 4 along N; wave (wm, wn) owns 64 rows
// x NB n-blocks of 16 columns = 4 x NB MFMA tiles (NB = 4 for q1 / tq2,
// 128 x 256 tiles; 2 for tq5, 128 x 128 tiles), so every decoded weight
// operand feeds 4 MFMAs.
//
// Activations: a ring of three LDS stages, each one group of the tile (128
// tokens x 128 k, 32 KB) in the order the MFMA reads it: 1 KB blocks, one
// per (16-row block, k-step), with lane 16q + j's 16 bytes at 16 * lane.
// Direct global-to-LDS loads (global_load_lds_dwordx4: each lane's 16 bytes
// land at 16 * lane from the block base) fill stage (i + 2) while stage i is
// multiplied; every wave issues the same number XB = 16 / NWN of them per
// group, last among its loads of the group, so waiting until at most XB
// loads are outstanding means the stage needed next has arrived.
//
// Work split (stream-K): the (tile, group) items, tiles ordered token tile
// fastest, are cut into one contiguous range per workgroup slot of the chip.
// A tile whose groups a range covers entirely is stored directly; the pieces
// of a split tile go to the caller's workspace as agent-scope atomic stores,
// one arrival counter per tile (zero between calls) tells the last of its
// workgroups, which adds the pieces in K order (so the result does not
// depend on arrival order), writes Y and resets the counter.  Without a
// workspace every workgroup takes whole tiles.
//
// Ternary base-3 bytes (5 trits per byte) are decoded with a 243-entry LDS
// table giving the five (sign, non-zero) bit pairs of a byte at bits
// 15-2i / 14-2i; a shift by 2i and a mask then give the operand half 2t of
// trit i.  In a full 640-trit segment byte b carries trit i of group i at
// offset b, so one table lookup serves five groups; the bytes of the next
// segment are loaded two groups before it starts.
#include "device.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

constexpr int kBM = 128;
constexpr int kStages = 3;
// 8 waves, 4 side by side along N and two rows of them along M (two waves
// per SIMD).  A wave owns 64 rows x NB n-blocks of 16 columns: NB = 4 for
// q1 / tq2 (128 x 256 tiles), 2 for tq5 (128 x 128 tiles: its staged
// segment bytes grow with the tile width, and its decoded segment words
// with the wave's width).
template <int FMT>
constexpr int nwn() { return 4; }
template <int FMT>
constexpr int nbw() { return FMT == 3 ? 2 : 4; }
template <int FMT>
constexpr int threads_of() { return 128 * nwn<FMT>(); }
template <int FMT>
constexpr int bn_of() { return 16 * nbw<FMT>() * nwn<FMT>(); }
template <int FMT>
constexpr int piece_floats() { return 2 * nwn<FMT>() * 64 * 16 * nbw<FMT>(); }  // one tile, lane order
constexpr int kStageBytes = kBM * 128 * 2;  // one group of the activation tile
constexpr int64_t kCounterBytes = 64 << 10;  // arrival counters (up to 16384 tiles)
constexpr int kRawBytes = 16 << 10;          // tq5 raw segment bytes per stage

struct GemmParams {
  const uint8_t *W;
  const uint8_t *Sc;  // plane B (may be only 2-byte aligned for tq5)
  const uint16_t *X;
  const uint8_t *XP;  // fp8 x pieces (q1, bf16 x): [tile_m][group] 32 KB blocks
  const uint8_t *XS;  // their E8M0 scales: [tile_m][group][row block] 64 bytes
  void *Y;
  float *part;      // [slot][2] pieces of split tiles (stream-K)
  unsigned *count;  // [tiles] arrival counters
  int M, N, K, G;
  int tiles_m, tiles_n;
  int64_t items;  // tiles * G
  int per;        // items per workgroup
  int last_chunk_groups;  // groups in the last chunk of 4 (1..4)
  int y_f16;
  // tq5 geometry
  int s_full, L_tail, b_tail, rowbytes;
};

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

typedef __attribute__((address_space(3))) void lds_void;

struct TileCols {
  int tileT[4], RT[4];
};

template <int FMT>
__device__ __forceinline__ TileCols tile_cols(const GemmParams &p, int nt) {
  const int wn = uni(threadIdx.x >> 6) % nwn<FMT>();
  TileCols c;
#pragma unroll
  for (int nb = 0; nb < nbw<FMT>(); ++nb) {
    const int n = nt * bn_of<FMT>() + wn * 16 * nbw<FMT>() + 16 * nb;
    c.tileT[nb] = uni(n / 16);
    c.RT[nb] = uni(n < p.N ? min(16, p.N - n) : 0);
  }
  return c;
}

// Row tile and rows of n-block nb of column half wn of column tile nt, by
// arithmetic (a runtime index into a per-thread array would put it in
// scratch memory).  Blocks past N get tile 0 with one row: an in-bounds
// address whose loads feed only unstored columns.
struct ColBlock {
  int T, R, RR;
};

template <int FMT>
__device__ __forceinline__ ColBlock col_block(const GemmParams &p, int nt, int wn, int nb) {
  const int n = nt * bn_of<FMT>() + wn * 16 * nbw<FMT>() + 16 * nb;
  ColBlock c;
  c.R = n < p.N ? min(16, p.N - n) : 0;
  c.T = c.R > 0 ? n / 16 : 0;
  c.RR = c.R > 0 ? c.R : 1;
  return c;
}

// Per-item weight staging (in the same LDS ring as the activations): the
// packed words of the tile's columns -- [wn][nb][word][lane] x 4 bytes,
// one word per lane for q1, two for tq2 -- and their FP16 scales at
// [wave][lane] x 4 bytes (a 2-byte global-to-LDS load writes its lane's
// value zero-extended at 4 * lane; lane l carries the scale of row l % 16 of
// n-block H wm + (l / 16) % H, H = NB / 2).  Wave (wm, wn) loads n-blocks
// H wm .. H wm + H - 1 of its column block.  Weight rows past N (ragged last
// tile, n-blocks past N) read a clamped, in-bounds address and keep whatever
// they load: they only feed output columns that are never stored.
template <int FMT>
constexpr int w_words() { return FMT == 2 ? 2 : (FMT == 1 ? 1 : 0); }

template <int FMT>
constexpr int w_scale_off() { return nwn<FMT>() * nbw<FMT>() * w_words<FMT>() * 256; }

template <int FMT>
constexpr int w_raw_off() { return w_scale_off<FMT>() + 2 * nwn<FMT>() * 256; }

// q1 with fp8 x pieces: the item's 512 E8M0 x scales (8 row blocks x 64).
template <int FMT>
constexpr int w_xscale_off() { return w_raw_off<FMT>() + (FMT == 3 ? kRawBytes : 0); }

template <int FMT>
constexpr int w_stage_bytes() {
  return w_xscale_off<FMT>() + (FMT == 1 ? 512 : 0);
}

template <int FMT>
__device__ __forceinline__ float w_scale(const char *wst, int nb) {
  constexpr int H = nbw<FMT>() / 2;  // n-blocks whose scales one wave stages
  const int wn = (threadIdx.x >> 6) % nwn<FMT>(), j = threadIdx.x & 15;
  const int wave = (nb / H) * nwn<FMT>() + wn;
  const uint16_t h =
      *reinterpret_cast<const uint16_t *>(wst + w_scale_off<FMT>() + wave * 256 + ((nb % H) * 16 + j) * 4);
  return half_to_float(h);
}

template <int FMT>
__device__ __forceinline__ uint32_t w_word(const char *wst, int nb, int h) {
  const int wn = (threadIdx.x >> 6) % nwn<FMT>(), lane = threadIdx.x & 63;
  return *reinterpret_cast<const uint32_t *>(wst + ((wn * nbw<FMT>() + nb) * w_words<FMT>() + h) * 256 + lane * 4);
}

// 4 k-steps of MFMAs for one group from stage st into fresh tiles, then
// acc += s * tile.  Bop(u, nb) returns the B operand (16 weight rows x 32 k)
// of n-block nb for k-step u.
template <int FMT, bool BF, class Bop>
__device__ __forceinline__ void group_mma(const char *st, const float (&sc)[nbw<FMT>()], f4_t (&acc)[4][nbw<FMT>()],
                                          Bop bop) {
  constexpr int NB = nbw<FMT>();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / nwn<FMT>();
  f4_t cg[4][NB];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    u4_t A[4], B[NB];
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
      A[mb] = *reinterpret_cast<const u4_t *>(st + ((wm * 4 + mb) * 4 + u) * 1024 + lane * 16);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) B[nb] = bop(u, nb);
#pragma unroll
    for (int mb = 0; mb < 4; ++mb)
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
        cg[mb][nb] = u == 0 ? mfma16x16x32_zero<BF>(A[mb], B[nb]) : mfma16x16x32<BF>(A[mb], B[nb], cg[mb][nb]);
  }
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < NB; ++nb)
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[mb][nb][e] = fmaf(sc[nb], cg[mb][nb][e], acc[mb][nb][e]);
}

// q1 with fp8 x pieces: one group on v_mfma_scale_f32_16x16x128_f8f6f4.
// Row block mb of stage st is four 1 KB blocks (hi piece halves 0 and 1, lo
// piece halves 0 and 1; lane l's 16 bytes at 16 l), its E8M0 scales 64
// bytes of the weight stage (lane 16 kb + r: row r, k-block kb).  The
// weights decode to fp4 +-1 (q1_fp4) once per n-block; the hi and lo MFMAs
// of a (row block, n-block) chain into one fresh tile that is added as
// s * tile, as in the bf16 path.
template <int FMT>
__device__ __forceinline__ void group_mma_xp(const char *st, const char *wst, const float (&sc)[nbw<FMT>()],
                                             const uint32_t (&wd)[nbw<FMT>()][2], f4_t (&acc)[4][nbw<FMT>()]) {
  constexpr int NB = nbw<FMT>();
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / nwn<FMT>();
  u4_t b[NB];
#pragma unroll
  for (int nb = 0; nb < NB; ++nb) b[nb] = q1_fp4(wd[nb][0]);
#pragma unroll
  for (int mb = 0; mb < 4; ++mb) {
    const int rb = wm * 4 + mb;
    const char *blk = st + rb * 4096 + lane * 16;
    const u4_t h0 = *reinterpret_cast<const u4_t *>(blk);
    const u4_t h1 = *reinterpret_cast<const u4_t *>(blk + 1024);
    const u4_t l0 = *reinterpret_cast<const u4_t *>(blk + 2048);
    const u4_t l1 = *reinterpret_cast<const u4_t *>(blk + 3072);
    const int sa = *reinterpret_cast<const uint8_t *>(wst + w_xscale_off<FMT>() + rb * 64 + lane);
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) {
      const f4_t d = mfma_f8f4_acc(l0, l1, b[nb], sa, mfma_f8f4(h0, h1, b[nb], sa));
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[mb][nb][e] = fmaf(sc[nb], d[e], acc[mb][nb][e]);
    }
  }
}

template <int FMT>
__device__ __forceinline__ void store_tile(const GemmParams &p, int mt, int nt, const f4_t (&acc)[4][nbw<FMT>()]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wm = wave / nwn<FMT>(), wn = wave % nwn<FMT>();
  const int j = lane & 15, q = lane >> 4;
  const float mul = FMT == 1 ? 1.f : 0.5f;  // ternary operands carry 2t
#pragma unroll
  for (int mb = 0; mb < 4; ++mb)
#pragma unroll
    for (int nb = 0; nb < nbw<FMT>(); ++nb) {
      const int n = nt * bn_of<FMT>() + wn * 16 * nbw<FMT>() + 16 * nb + j;
      if (n >= p.N) continue;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        const int m = mt * kBM + wm * 64 + 16 * mb + 4 * q + e;
        if (m >= p.M) continue;
        const float v = acc[mb][nb][e] * mul;
        if (p.y_f16) reinterpret_cast<uint16_t *>(p.Y)[(int64_t)m * p.N + n] = float_to_half_rne(v);
        else reinterpret_cast<float *>(p.Y)[(int64_t)m * p.N + n] = v;
      }
    }
}

// tq5: the raw bytes of the full segment holding each item, staged on the
// items that decode them, in the weight stage (after the scales): layout
// [wn][nb][half][lane] x 16 bytes (32 bytes per lane and n-block, 16 KB);
// wave (wm, wn) fills n-block wm of its column block.

// (sign, non-zero) pairs of the segment for the wave's 4 n-blocks, from the
// staged raw bytes through the 243-entry table.
__device__ __forceinline__ void tq5_decode(const char *slot, const uint16_t *lut, uint32_t (&d5)[nbw<3>()][16]) {
  const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
  const int wn = wave % nwn<3>();
#pragma unroll
  for (int nb = 0; nb < nbw<3>(); ++nb) {
    const u4_t a = *reinterpret_cast<const u4_t *>(slot + ((wn * nbw<3>() + nb) * 2 + 0) * 1024 + lane * 16);
    const u4_t b = *reinterpret_cast<const u4_t *>(slot + ((wn * nbw<3>() + nb) * 2 + 1) * 1024 + lane * 16);
    const uint32_t wds[8] = {a.x, a.y, a.z, a.w, b.x, b.y, b.z, b.w};
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

// The stream of items this workgroup loads, two ahead of the one it
// multiplies: position (tile, group), the tile's coordinates and the lane
// addresses that depend only on the tile (refreshed when the tile changes),
// so that issuing an item's loads is a few adds per load.
template <int FMT>
struct Feed {
  int tile, g, mt, nt;
  const uint16_t *xrow[2];  // activation rows of the wave's row blocks (+ 8q), see x_blocks
  const uint8_t *wb[2];     // n-blocks H wm + i the wave loads: tile block start (tq5: + lane part)
  uint32_t wl[2];           // q1: 4 woff, tq2: 8 woff (woff = lane word index q RR + j)
  int RR[2];                // rows of the block (>= 1)
  const uint8_t *sctile;    // plane B start of this lane's scale tile
  int sRR, sjj;             // that tile's rows, this lane's row in it
};

// Activation blocks (16 rows x one k-step, 1 KB) each wave loads per item:
// the 32 blocks of a group split over the 2 * nwn waves; wave w takes blocks
// w * XB .. w * XB + XB - 1 (row block b / 4, k-step b % 4).
template <int FMT>
constexpr int x_blocks() { return 32 / (2 * nwn<FMT>()); }

template <int FMT>
__device__ __forceinline__ void feed_tile(const GemmParams &p, Feed<FMT> &f) {
  constexpr int XB = x_blocks<FMT>();
  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int wm = wave / nwn<FMT>(), wn = wave % nwn<FMT>();
  const int j = lane & 15, q = lane >> 4;
#pragma unroll
  for (int h = 0; h < XB / 4; ++h)
    f.xrow[h] = p.X + (int64_t)min(f.mt * kBM + 16 * (wave * (XB / 4) + h) + j, p.M - 1) * p.K + 8 * q;
#pragma unroll
  for (int i = 0; i < nbw<FMT>() / 2; ++i) {
    const ColBlock cb = col_block<FMT>(p, f.nt, wn, (nbw<FMT>() / 2) * wm + i);
    const uint32_t woff = uint32_t(q * cb.RR + min(j, cb.RR - 1));
    f.RR[i] = cb.RR;
    if constexpr (FMT == 3) {
      f.wb[i] = p.W + 16 * (int64_t)cb.T * p.rowbytes + woff * 16;
    } else if constexpr (FMT == 1) {
      // word of (lane, group gc) in chunk c of Gc groups:
      // c * RR * 64 + 4 * (woff * Gc + gc) bytes
      f.wb[i] = p.W + 16 * (int64_t)cb.T * p.G * 16;
      f.wl[i] = 4 * woff;
    } else {
      // word pair of (lane, group gc) in chunk c, half hh = gc / 2 of Gh
      // groups: c * RR * 128 + hh * RR * 64 + 8 * (woff * Gh + gc - 2 hh) bytes
      f.wb[i] = p.W + 16 * (int64_t)cb.T * p.G * 32;
      f.wl[i] = 8 * woff;
    }
  }
  const ColBlock cs = col_block<FMT>(p, f.nt, wn, (nbw<FMT>() / 2) * wm + ((lane >> 4) % (nbw<FMT>() / 2)));
  f.sctile = p.Sc + 32 * (int64_t)cs.T * p.G;
  f.sRR = cs.RR;
  f.sjj = min(j, cs.RR - 1);
}

template <int FMT>
__device__ __forceinline__ void feed_next(const GemmParams &p, Feed<FMT> &f) {
  if (++f.g == p.G) {
    f.g = 0;
    ++f.tile;
    if (++f.mt == p.tiles_m) {
      f.mt = 0;
      ++f.nt;
    }
    feed_tile<FMT>(p, f);
  }
}

// All loads of item f into activation stage xst and weight stage wst:
// weights first, then the XB activation loads of the wave.  tq5 loads the
// raw bytes of a segment only with `raw` (the item that decodes them).  XP:
// the activations are the item's 32 KB block of fp8 x pieces (the same 32
// 1 KB blocks per item), and waves 0 and 1 first load its 512 x scales.
template <int FMT, bool XP>
__device__ __forceinline__ void feed_issue(const GemmParams &p, const Feed<FMT> &f, char *xst, char *wst, bool raw) {
  constexpr int XB = x_blocks<FMT>();
  const int wave = uni(threadIdx.x >> 6);
  const int wm = wave / nwn<FMT>(), wn = wave % nwn<FMT>();
  const int g = f.g;
  if constexpr (FMT != 3) {
    const int c = g >> 2, gc = g & 3;
    const int Gc = 4 * c + 4 > p.G ? p.last_chunk_groups : 4;
    const int hh = gc >> 1;
    const int Gh = min(2, Gc - 2 * hh);
#pragma unroll
    for (int i = 0; i < nbw<FMT>() / 2; ++i) {
      const int nb = (nbw<FMT>() / 2) * wm + i;
      if constexpr (FMT == 1) {
        const uint8_t *a = f.wb[i] + (f.RR[i] * 64 * c + 4 * gc) + f.wl[i] * uint32_t(Gc);
        __builtin_amdgcn_global_load_lds((const void *)a, (lds_void *)(wst + (wn * nbw<FMT>() + nb) * 256), 4, 0, 0);
      } else {
        const uint8_t *a = f.wb[i] + (f.RR[i] * (128 * c + 64 * hh) + 8 * (gc - 2 * hh)) + f.wl[i] * uint32_t(Gh);
        __builtin_amdgcn_global_load_lds((const void *)a, (lds_void *)(wst + ((wn * nbw<FMT>() + nb) * 2) * 256), 4,
                                         0, 0);
        __builtin_amdgcn_global_load_lds((const void *)(a + 4),
                                         (lds_void *)(wst + ((wn * nbw<FMT>() + nb) * 2 + 1) * 256), 4, 0, 0);
      }
    }
  }
  // Plane B: chunk sc of W groups (4; tq5: its 5-group segments) starts at
  // RR W sc in the tile, the lane's row at sjj Gs.
  constexpr int W = FMT == 3 ? 5 : 4;
  const int sc = g / W, gs = g - W * sc, Gs = min(W, p.G - W * sc);
  __builtin_amdgcn_global_load_lds((const void *)(f.sctile + 2 * (f.sRR * W * sc + f.sjj * Gs + gs)),
                                   (lds_void *)(wst + w_scale_off<FMT>() + wave * 256), 2, 0, 0);
  if constexpr (FMT == 3) {
    const int seg = g / 5;
    if (raw && seg < p.s_full) {  // wave-uniform
      char *slot = wst + w_raw_off<FMT>();
#pragma unroll
      for (int i = 0; i < nbw<FMT>() / 2; ++i) {
        const int nb = (nbw<FMT>() / 2) * wm + i;
        const uint8_t *sb = f.wb[i] + (int64_t)f.RR[i] * 128 * seg;
#pragma unroll
        for (int h = 0; h < 2; ++h)
          __builtin_amdgcn_global_load_lds((const void *)(sb + h * f.RR[i] * 64),
                                           (lds_void *)(slot + ((wn * nbw<FMT>() + nb) * 2 + h) * 1024), 16, 0, 0);
      }
    }
  }
  if constexpr (XP) {
    const int lane = threadIdx.x & 63;
    const int64_t item = (int64_t)f.mt * p.G + g;
    if (wave < 2)
      __builtin_amdgcn_global_load_lds((const void *)(p.XS + item * 512 + wave * 256 + lane * 4),
                                       (lds_void *)(wst + w_xscale_off<FMT>() + wave * 256), 4, 0, 0);
    const uint8_t *xb = p.XP + item * 32768 + lane * 16;
#pragma unroll
    for (int i = 0; i < XB; ++i)
      __builtin_amdgcn_global_load_lds((const void *)(xb + (wave * XB + i) * 1024),
                                       (lds_void *)(xst + (wave * XB + i) * 1024), 16, 0, 0);
  } else {
#pragma unroll
    for (int i = 0; i < XB; ++i)
      __builtin_amdgcn_global_load_lds((const void *)(f.xrow[i >> 2] + 128 * g + 32 * (i & 3)),
                                       (lds_void *)(xst + (wave * XB + i) * 1024), 16, 0, 0);
  }
}

template <int FMT, bool BF, bool XP>
__global__ void __launch_bounds__(threads_of<FMT>()) gemm_kernel(GemmParams p) {
  extern __shared__ __align__(16) char xs[];  // kStages x (activations, then weights)
  __shared__ uint16_t lut[256];
  __shared__ int last_flag;
  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int j = lane & 15, q = lane >> 4;

  if constexpr (FMT == 3) {
    for (int v = threadIdx.x; v < 256; v += threads_of<FMT>()) {
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

  const int G = p.G;
  // This workgroup's items [i0, i0 + n): whole tile blockIdx.x, or (stream-K,
  // fewer than 2^31 items) a range of per items.  wf / wl: the workgroups
  // whose ranges cover the first and the last tile of the range (only those
  // two tiles can be split between workgroups).
  int n, first_tile, last_tile, g0, wf0, wl0, wf1, wl1;
  if (p.per == G) {
    n = G;
    first_tile = last_tile = blockIdx.x;
    g0 = 0;
    wf0 = wl0 = wf1 = wl1 = blockIdx.x;
  } else {
    const uint32_t per = uint32_t(p.per), ug = uint32_t(G);
    const uint32_t i0 = blockIdx.x * per;
    const uint32_t i1 = min(i0 + per, uint32_t(p.items));
    if (i0 >= i1) return;  // workgroup-uniform
    n = int(i1 - i0);
    first_tile = int(i0 / ug);
    last_tile = int((i1 - 1) / ug);
    g0 = int(i0 - uint32_t(first_tile) * ug);
    wf0 = int(uint32_t(first_tile) * ug / per);
    wl0 = int((uint32_t(first_tile) * ug + ug - 1) / per);
    wf1 = int(uint32_t(last_tile) * ug / per);
    wl1 = int((uint32_t(last_tile) * ug + ug - 1) / per);
  }

  constexpr int NB = nbw<FMT>();
  f4_t acc[4][NB];
  int cur_tile = first_tile, cur_g = g0;
  int cur_mt = first_tile % p.tiles_m, cur_nt = first_tile / p.tiles_m;
  int g_begin = cur_g;
  TileCols tc = tile_cols<FMT>(p, cur_nt);

  // tq5: decoded pairs of the current segment.
  uint32_t d5[NB][16];
  char *wring = xs + kStages * kStageBytes;  // weight stages (kStages x w_stage_bytes)
  constexpr int kW = w_stage_bytes<FMT>();

  // Items 0 and 1 in flight; the feed then points at item 2 (it stops at
  // the last item, whose loads are repeated into otherwise unused stages).
  Feed<FMT> feed;
  feed.tile = cur_tile;
  feed.g = cur_g;
  feed.mt = cur_mt;
  feed.nt = cur_nt;
  feed_tile<FMT>(p, feed);
  int feed_it = 0;
  auto raw_for = [&]() { return FMT == 3 && (feed_it == 0 || feed.g % 5 == 0); };
  feed_issue<FMT, XP>(p, feed, xs, wring, raw_for());
  if (feed_it + 1 < n) { feed_next<FMT>(p, feed); ++feed_it; }
  feed_issue<FMT, XP>(p, feed, xs + kStageBytes, wring + kW, raw_for());
  if (feed_it + 1 < n) { feed_next<FMT>(p, feed); ++feed_it; }

  auto step = [&](int it, int slot) {
    const int tile = cur_tile, g = cur_g, mt = cur_mt, nt = cur_nt;
    if (++cur_g == G) {
      cur_g = 0;
      ++cur_tile;
      if (++cur_mt == p.tiles_m) {
        cur_mt = 0;
        ++cur_nt;
      }
    }
    const bool first = it == 0 || g == 0;
    const bool last = it == n - 1 || g == G - 1;
    if (first) {
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b) acc[a][b] = f4_t{0.f, 0.f, 0.f, 0.f};
      if constexpr (FMT == 3) tc = tile_cols<FMT>(p, nt);
      g_begin = g;
    }
    // Stage `slot` holds item it once at most the XB activation loads of
    // item it + 1 are outstanding (the last item waits for all).
    if (it + 1 < n) __builtin_amdgcn_s_waitcnt(0x0F70 | x_blocks<FMT>());  // vmcnt(XB)
    else __builtin_amdgcn_s_waitcnt(0x0F70);                            // vmcnt(0)
    // A plain barrier: __syncthreads() would also wait for every global load
    // in flight.  LDS here is written only by the staging loads waited for
    // above, and this wave's reads of the stage refilled below were consumed
    // by its MFMAs of the previous item.
    __builtin_amdgcn_s_barrier();
    feed_issue<FMT, XP>(p, feed, xs + ((slot + 2) % kStages) * kStageBytes, wring + ((slot + 2) % kStages) * kW,
                    raw_for());
    if (feed_it + 1 < n) { feed_next<FMT>(p, feed); ++feed_it; }
    const char *st = xs + slot * kStageBytes;
    const char *wst = wring + slot * kW;
    float sc[NB];
#pragma unroll
    for (int nb = 0; nb < NB; ++nb) sc[nb] = w_scale<FMT>(wst, nb);
    if constexpr (FMT != 3) {
      uint32_t wd[NB][2];
#pragma unroll
      for (int nb = 0; nb < NB; ++nb)
#pragma unroll
        for (int h = 0; h < w_words<FMT>(); ++h) wd[nb][h] = w_word<FMT>(wst, nb, h);
      if constexpr (XP) {
        group_mma_xp<FMT>(st, wst, sc, wd, acc);
      } else {
        group_mma<FMT, BF>(st, sc, acc, [&](int u, int nb) -> u4_t {
          if constexpr (FMT == 1) return q1_operand_pm1<BF>(wd[nb][0], u);
          else return tq2_operand(wd[nb][u >> 1], u);
        });
      }
    } else {
      const int seg = g / 5, gs = g - 5 * seg;
      if (seg < p.s_full) {
        if (gs == 0 || first) tq5_decode(wst + w_raw_off<FMT>(), lut, d5);
        group_mma<FMT, BF>(st, sc, acc, [&](int u, int nb) -> u4_t {
          u4_t b;
          b.x = tq5_pair(d5[nb][u * 4 + 0], gs);
          b.y = tq5_pair(d5[nb][u * 4 + 1], gs);
          b.z = tq5_pair(d5[nb][u * 4 + 2], gs);
          b.w = tq5_pair(d5[nb][u * 4 + 3], gs);
          return b;
        });
      } else {
        // Tail segment, row-major bytes: offset kt -> byte kt % B, digit kt / B.
        group_mma<FMT, BF>(st, sc, acc, [&](int u, int nb) -> u4_t {
          uint32_t h[8];
          const int R = tc.RT[nb];
          const int jj = min(j, max(R - 1, 0));
          const int T = R > 0 ? tc.tileT[nb] : 0;
          const int RR = R > 0 ? R : 1;
          const uint8_t *tb = p.W + 16 * (int64_t)T * p.rowbytes + (int64_t)RR * 128 * p.s_full + (int64_t)jj * p.b_tail;
#pragma unroll
          for (int e = 0; e < 8; ++e) {
            const int kt = 128 * (g - 5 * p.s_full) + 32 * u + 8 * q + e;
            const int b = kt % p.b_tail, dig = kt / p.b_tail;
            int v = tb[b];
            for (int t = 0; t < dig; ++t) v /= 3;
            const int d = v % 3;
            h[e] = d == 1 ? 0u : (d == 2 ? 0x4000u : 0xC000u);
          }
          u4_t b;
          b.x = h[0] | (h[1] << 16);
          b.y = h[2] | (h[3] << 16);
          b.z = h[4] | (h[5] << 16);
          b.w = h[6] | (h[7] << 16);
          return b;
        });
      }
    }
    if (!last) return;
    if (g_begin == 0 && g == G - 1) {  // whole tile in this range
      store_tile<FMT>(p, mt, nt, acc);
      return;
    }
    // Split tile: publish this piece (slot 0: this range's first tile, 1: its last).
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
    const int which = tile == first_tile ? 0 : 1;
    const int wf = which ? wf1 : wf0, wl = which ? wl1 : wl0;
    float *piece = p.part + ((int64_t)blockIdx.x * 2 + which) * piece_floats<FMT>();
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b)
#pragma unroll
        for (int e = 0; e < 4; ++e)
          __hip_atomic_store(piece + ((wave * 4 * NB + a * NB + b) * 4 + e) * 64 + lane, acc[a][b][e], __ATOMIC_RELAXED,
                             __HIP_MEMORY_SCOPE_AGENT);
    __builtin_amdgcn_s_waitcnt(0);  // this thread's piece stores have completed
    __syncthreads();
    if (threadIdx.x == 0)
      last_flag = __hip_atomic_fetch_add(p.count + tile, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) ==
                  unsigned(wl - wf);
    __syncthreads();
    if (!last_flag) return;
    f4_t sum[4][NB];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
      for (int b = 0; b < NB; ++b) sum[a][b] = f4_t{0.f, 0.f, 0.f, 0.f};
    for (int w2 = wf; w2 <= wl; ++w2) {
      // Piece 0 of workgroup w2 belongs to the first tile of its range.
      const int wh = int(uint32_t(w2) * uint32_t(p.per) / uint32_t(G)) == tile ? 0 : 1;
      const float *pc = p.part + ((int64_t)w2 * 2 + wh) * piece_floats<FMT>();
#pragma unroll
      for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < NB; ++b)
#pragma unroll
          for (int e = 0; e < 4; ++e)
            sum[a][b][e] += __hip_atomic_load(pc + ((wave * 4 * NB + a * NB + b) * 4 + e) * 64 + lane, __ATOMIC_RELAXED,
                                              __HIP_MEMORY_SCOPE_AGENT);
    }
    store_tile<FMT>(p, mt, nt, sum);
    if (threadIdx.x == 0) __hip_atomic_store(p.count + tile, 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
  };

  for (int it = 0; it < n; it += 3) {
    step(it, 0);
    if (it + 1 >= n) break;
    step(it + 1, 1);
    if (it + 2 >= n) break;
    step(it + 2, 2);
  }
}

int stream_k_slots() { return num_cus(); }

// fp8 x pieces for the q1 GEMM with bf16 x, converted once per launch:
// thread = item (row m of the padded token tiles, group g, lane quarter q),
// the 32 values x[m][128 g + 32 u + 8 q + e] (u < 4, e < 8) as two e4m3
// pieces and one E8M0 scale (split_x_quarter; rows past M are zeros).  They
// form k-block q of the A operand of row r = m % 16 in row block mb =
// (m % 128) / 16 of token tile mt: the first 16 bytes of each piece go to
// lane 16 (2 (q & 1)) + r, the second 16 to the lane 16 above it, both in
// half q / 2 of that lane's 32 bytes; the scale is byte 16 q + r of the row
// block's 64.  Layout: XP [mt][g][mb][piece][half] 1 KB blocks (lane l at
// 16 l), XS [mt][g][mb] 64 bytes.  A wave takes the 64 items (q, r) of one
// (mt, g, mb), so each of its stores fills whole 256-byte runs.
__global__ void x_pieces_kernel(const uint16_t *X, int M, int K, int G, int64_t items, uint8_t *XP, uint8_t *XS) {
  const int64_t item = blockIdx.x * (int64_t)blockDim.x + threadIdx.x;
  if (item >= items) return;
  const int r = int(item & 15), q = int((item >> 4) & 3);
  const int64_t rest = item >> 6;
  const int mb = int(rest & 7);
  const int64_t blk = rest >> 3;  // mt * G + g
  const int g = int(blk % G), mt = int(blk / G);
  const int m = mt * 128 + mb * 16 + r;
  const bool in = m < M;
  XQuarter xq;
  split_x_quarter<1>(X + (in ? (int64_t)m * K + 128 * g + 8 * q : 0), in, xq);
  uint8_t *b = XP + blk * 32768 + mb * 4096 + (q >> 1) * 1024;
  const int l0 = 16 * (2 * (q & 1)) + r, l1 = l0 + 16;
  *reinterpret_cast<u4_t *>(b + l0 * 16) = xq.h0;
  *reinterpret_cast<u4_t *>(b + l1 * 16) = xq.h1;
  *reinterpret_cast<u4_t *>(b + 2048 + l0 * 16) = xq.l0;
  *reinterpret_cast<u4_t *>(b + 2048 + l1 * 16) = xq.l1;
  XS[(blk * 8 + mb) * 64 + 16 * q + r] = xq.sb;
}

int64_t x_pieces_bytes(int64_t M, int64_t K) {
  return (M + kBM - 1) / kBM * (K / kGroup) * (32768 + 512);
}

// Workspace offset of the x pieces: after the stream-K counters and pieces.
template <int FMT>
int64_t x_pieces_offset() {
  return (kCounterBytes + (int64_t)stream_k_slots() * 2 * piece_floats<FMT>() * 4 + 255) / 256 * 256;
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
  p.last_chunk_groups = p.G - 4 * ((p.G - 1) / 4);
  p.tiles_n = int((a.N + bn_of<FMT>() - 1) / bn_of<FMT>());
  p.y_f16 = a.y_f16;
  const Tq5Geom t = tq5_geom(a.K);
  p.s_full = int(t.s_full); p.L_tail = int(t.L_tail); p.b_tail = int(t.b_tail); p.rowbytes = int(t.rowbytes);
  const int64_t tiles = (int64_t)p.tiles_m * p.tiles_n;
  p.items = tiles * p.G;
  const int slots = stream_k_slots();
  int grid;
  const bool sk = a.ws && tiles <= kCounterBytes / 4 && tiles > slots / 2 && p.items < (int64_t(1) << 31) &&
                  a.ws_bytes >= kCounterBytes + (int64_t)slots * 2 * piece_floats<FMT>() * 4;
  if (sk) {
    p.per = int((p.items + slots - 1) / slots);
    grid = int((p.items + p.per - 1) / p.per);
    p.count = static_cast<unsigned *>(a.ws);
    p.part = reinterpret_cast<float *>(static_cast<char *>(a.ws) + kCounterBytes);
  } else {
    p.per = p.G;  // whole tiles
    grid = int(tiles);
  }
  const int lds = kStages * (kStageBytes + w_stage_bytes<FMT>());
  if (a.plan) {
    lowbit_plan &o = plan_record(a, LOWBIT_KERNEL_GEMM, grid, threads_of<FMT>(), lds);
    o.token_slots = kBM;
    o.operands = BF ? LOWBIT_OPERANDS_BF16 : LOWBIT_OPERANDS_F16;
    o.tiles_per_wave = nbw<FMT>();
    o.ring = kStages;
    o.items_per_wg = p.per;
    if constexpr (FMT == 1 && BF) {
      if (a.ws && a.ws_bytes >= x_pieces_offset<FMT>() + x_pieces_bytes(a.M, a.K)) {
        o.x_pieces = 1;
        o.launches = 2;
        o.operands = LOWBIT_OPERANDS_FP8_FP4;
      }
    }
    return hipSuccess;
  }
  if constexpr (FMT == 1 && BF) {
    // Binary weights with bf16 x: x enters as fp8 pieces when the workspace
    // holds them (exact enough for binary weights: see the GEMV split path).
    const int64_t off = x_pieces_offset<FMT>();
    if (a.ws && a.ws_bytes >= off + x_pieces_bytes(a.M, a.K)) {
      p.XP = static_cast<const uint8_t *>(a.ws) + off;
      p.XS = p.XP + (int64_t)p.tiles_m * p.G * 32768;
      const int64_t items = (int64_t)p.tiles_m * kBM * p.G * 4;
      hipLaunchKernelGGL(x_pieces_kernel, dim3(unsigned((items + 255) / 256)), dim3(256), 0, a.stream, p.X, p.M,
                         p.K, p.G, items, const_cast<uint8_t *>(p.XP), const_cast<uint8_t *>(p.XS));
      hipLaunchKernelGGL((gemm_kernel<FMT, BF, true>), dim3(grid), dim3(threads_of<FMT>()), lds, a.stream, p);
      return hipGetLastError();
    }
  }
  hipLaunchKernelGGL((gemm_kernel<FMT, BF, false>), dim3(grid), dim3(threads_of<FMT>()), lds, a.stream, p);
  return hipGetLastError();
}

}  // namespace

int64_t gemm_workspace_bytes(int fmt, int64_t M, int64_t N, int64_t K) {
  (void)N;
  if (fmt == 1) return x_pieces_offset<1>() + x_pieces_bytes(M, K);  // + fp8 x pieces (bf16 x)
  const int64_t piece = fmt == 3 ? piece_floats<3>() : piece_floats<1>();
  return kCounterBytes + (int64_t)stream_k_slots() * 2 * piece * 4;
}

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
