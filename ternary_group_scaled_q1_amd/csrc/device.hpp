// Device-side helpers shared by the GEMV and GEMM kernels (gfx950 / CDNA4).
//
// Decode strategy.  The matrix cores multiply 16x32 by 32x16 f16/bf16 tiles
// (v_mfma_f32_16x16x32_{f16,bf16}); a lane supplies 8 halves of one operand
// row/column.  The packed weights are turned into exact operand halves with
// a shift and one bitwise op per pair of weights:
//  * q1 "sign" pairs: the two weight bits sit at 15/31 -> (E & 0x80008000) ^ (-1,-1)
//    gives +1 for bit 1 and -1 for bit 0 (stored bit 1 means +scale);
//  * q1 "plus-one" pairs: bits at 14/30 -> E & 0x40004000 gives 2 for bit 1 and
//    0 for bit 0, i.e. t + 1; the extra +x is removed once per group;
//  * tq2 pairs: the 2-bit codes c = t + 1 sit at 14..15 / 30..31 ->
//    ~E & 0xC000C000 gives -2, -0, +2 for c = 0, 1, 2, i.e. exactly 2t.
// 2.0 is 0x4000 in both f16 and bf16, and +-1 differ only in the sign bit, so
// every operand half is exact; products with x are exact in the fp32
// accumulator.
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace lowbit {

typedef _Float16 h8_t __attribute__((ext_vector_type(8)));
typedef __bf16 b8_t __attribute__((ext_vector_type(8)));
typedef float f4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u2_t __attribute__((ext_vector_type(2)));

template <bool BF>
__device__ __forceinline__ f4_t mfma16x16x32(u4_t a, u4_t b, f4_t c) {
  if constexpr (BF)
    return __builtin_amdgcn_mfma_f32_16x16x32_bf16(__builtin_bit_cast(b8_t, a),
                                                   __builtin_bit_cast(b8_t, b), c, 0, 0, 0);
  else
    return __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(h8_t, a),
                                                  __builtin_bit_cast(h8_t, b), c, 0, 0, 0);
}

template <bool BF>
__device__ __forceinline__ f4_t mfma16x16x32_zero(u4_t a, u4_t b) {
  const f4_t z = {0.f, 0.f, 0.f, 0.f};
  return mfma16x16x32<BF>(a, b, z);
}

// Two -1.0 halves.
template <bool BF>
__device__ __forceinline__ constexpr uint32_t neg_one2() {
  return BF ? 0xBF80BF80u : 0xBC00BC00u;
}

// q1, k-step u of a lane word w: pairs (sign, plus-one, sign, plus-one).
template <bool BF>
__device__ __forceinline__ u4_t q1_operand(uint32_t w, int u) {
  const uint32_t e0 = w << (4 * u);
  const uint32_t e1 = w << (4 * u + 2);
  u4_t b;
  b.x = (e0 & 0x80008000u) ^ neg_one2<BF>();
  b.y = e0 & 0x40004000u;
  b.z = (e1 & 0x80008000u) ^ neg_one2<BF>();
  b.w = e1 & 0x40004000u;
  return b;
}

// q1 without the plus-one pairs: every pair becomes +-1 (one extra shift for
// the pairs stored at 14/30).  Used where a per-(token, group) correction
// would cost more than the shift (the GEMM).
template <bool BF>
__device__ __forceinline__ u4_t q1_operand_pm1(uint32_t w, int u) {
  const uint32_t e0 = w << (4 * u);
  u4_t b;
  b.x = (e0 & 0x80008000u) ^ neg_one2<BF>();
  b.y = ((e0 << 1) & 0x80008000u) ^ neg_one2<BF>();
  b.z = ((e0 << 2) & 0x80008000u) ^ neg_one2<BF>();
  b.w = ((e0 << 3) & 0x80008000u) ^ neg_one2<BF>();
  return b;
}

// tq2, k-step u: w is the lane word holding steps (u & ~1, u | 1).  Gives 2t.
__device__ __forceinline__ u4_t tq2_operand(uint32_t w, int u) {
  const int s0 = 8 * (u & 1);
  u4_t b;
  b.x = ~(w << (s0 + 0)) & 0xC000C000u;
  b.y = ~(w << (s0 + 2)) & 0xC000C000u;
  b.z = ~(w << (s0 + 4)) & 0xC000C000u;
  b.w = ~(w << (s0 + 6)) & 0xC000C000u;
  return b;
}

// tq5: d holds two 10-bit trit fields (lo/hi halves), field i at bits
// 15-2i (sign) and 14-2i (non-zero).  Gives 2t for group i of the segment.
__device__ __forceinline__ uint32_t tq5_pair(uint32_t d, int i) {
  return (d << (2 * i)) & 0xC000C000u;
}

// ---- Scaled fp8 x fp4 matrix path (v_mfma_scale_f32_16x16x128_f8f6f4) ----
//
// Lane layout of the 16x16x128 instruction (measured on gfx950):
//  * B, fp4 e2m1: lane 16q + j holds column j at k = 32q + n for its nibble n
//    (nibble n in dword n / 8, bits 4(n % 8) .. 4(n % 8) + 3);
//  * A, fp8 e4m3: lane 16q + r holds row r at k = 16q + b for bytes b < 16 and
//    at k = 64 + 16q + (b - 16) for bytes b >= 16;
//  * the E8M0 scale of lane 16kb + r (byte 0) multiplies row r of A (column r
//    of B) over k in [32kb, 32kb + 32);
//  * D lane 16q + j, element e: row 4q + e, column j.
// +-1 and +-2 are exact in fp4 e2m1, so a weight decodes to an exact operand.
typedef int i8v_t __attribute__((ext_vector_type(8)));

// A = x pieces (fp8), B = weights (fp4, scale 1), fresh fp32 accumulator.
__device__ __forceinline__ f4_t mfma_f8f4(u4_t a0, u4_t a1, u4_t b, int sa) {
  const i8v_t A = {int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
  const i8v_t B = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
  const f4_t z = {0.f, 0.f, 0.f, 0.f};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, z, 0, 4, 0, sa, 0, 0x7F7F7F7F);
}

// The same, added to the fp32 tile c.
__device__ __forceinline__ f4_t mfma_f8f4_acc(u4_t a0, u4_t a1, u4_t b, int sa, f4_t c) {
  const i8v_t A = {int(a0.x), int(a0.y), int(a0.z), int(a0.w), int(a1.x), int(a1.y), int(a1.z), int(a1.w)};
  const i8v_t B = {int(b.x), int(b.y), int(b.z), int(b.w), 0, 0, 0, 0};
  return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(A, B, c, 0, 4, 0, sa, 0, 0x7F7F7F7F);
}

// q1 word -> 32 fp4 weights: nibble i of dword d takes bit 4i + 3 - d;
// bit 1 -> +1.0 (0x2), bit 0 -> -1.0 (0xA).
__device__ __forceinline__ u4_t q1_fp4(uint32_t w) {
  u4_t b;
  b.x = (~w & 0x88888888u) | 0x22222222u;
  b.y = (~(w << 1) & 0x88888888u) | 0x22222222u;
  b.z = (~(w << 2) & 0x88888888u) | 0x22222222u;
  b.w = (~(w << 3) & 0x88888888u) | 0x22222222u;
  return b;
}

// tq2 words (two per lane and group) -> 32 fp4 values 2t: nibble i of dword d
// takes the code at bits 4i + 2 - 2(d % 2) of word d / 2; ~c at nibble bits
// 2..3 is 0xC (-2), 0x8 (-0) or 0x4 (+2) for c = 0, 1, 2.
__device__ __forceinline__ u4_t tq2_fp4(uint32_t w0, uint32_t w1) {
  u4_t b;
  b.x = ~w0 & 0xCCCCCCCCu;
  b.y = ~(w0 << 2) & 0xCCCCCCCCu;
  b.z = ~w1 & 0xCCCCCCCCu;
  b.w = ~(w1 << 2) & 0xCCCCCCCCu;
  return b;
}

// Which in-group weight (8u + e: k = 32u + 8q + e for lane quarter q) feeds
// fp4 nibble n of a lane's operand (the inverses of q1_fp4 / tq2_fp4 over the
// bit positions of device layout v2).
__device__ constexpr int fp4_src(int fmt, int n) {
  const int d = n / 8, i = n % 8;
  if (fmt == 1) {
    const int pbit = 4 * i + 3 - d;
    const int rem = 15 - pbit % 16;
    return 8 * (rem / 4) + (pbit / 16) + 2 * (rem % 2) + 4 * ((rem / 2) % 2);
  }
  const int pos = 4 * i + 2 - 2 * (d % 2);
  const int rem = 14 - pos % 16;
  return 8 * (2 * (d / 2) + rem / 8) + (pos / 16) + 2 * ((rem % 8) / 2);
}

// The 32 bf16 values of one lane quarter q of a group (k = 32u + 8q + e) as
// two fp8 pieces in nibble order: h0/l0 hold nibbles 0..15 and h1/l1 nibbles
// 16..31 (the A operand's hardware k 32q + n), sb the E8M0 scale.
struct XQuarter {
  u4_t h0, h1, l0, l1;
  uint8_t sb;
};

// Those 32 values are the 32 k of one E8M0 block of the B operand, so one
// scale S = 2^(sb - 127) covers them.  sb puts the block's largest magnitude
// in [128, 256) (below the fp8 maximum 448, so no piece can overflow); hi =
// fp8(x / S) and lo = fp8(x / S - hi), both rounded to nearest even.  A bf16
// value has 8 significant bits and each piece 4, so x = S (hi + lo) exactly
// unless x lies more than 2^10 below the block's largest value (then the
// error is below 2^-17 of it).  A block holding inf or nan gets the nan
// scale 0xFF.  x[u] holds the 8 values x[m][128 g + 32 u + 8 q .. + 8].
template <int FMT>
__device__ __forceinline__ void split_x_regs(const u4_t (&x)[4], XQuarter &o) {
  uint32_t v[16];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v[4 * u + 0] = x[u].x;
    v[4 * u + 1] = x[u].y;
    v[4 * u + 2] = x[u].z;
    v[4 * u + 3] = x[u].w;
  }
  // Largest magnitude: both halves of a word at once (packed 16-bit max).
  typedef unsigned short u2h_t __attribute__((ext_vector_type(2)));
  u2h_t m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u2h_t, v[i] & 0x7FFF7FFFu));
  const uint32_t mx = max(uint32_t(m2.x), uint32_t(m2.y));
  const int ef = int(mx >> 7);  // exponent field of the largest magnitude
  const int sb = ef == 255 ? 255 : max(ef - 7, 0);
  // S = 2^(sb - 127) as an f32 (2^-127 is a denormal).  The scaled
  // conversions of gfx950 divide by S on the way to fp8 and multiply by it
  // on the way back; each takes or gives two values, and a pair of bf16
  // goes to fp8 without a separate widening and scaling.
  const float S = sb == 0 ? __builtin_bit_cast(float, 0x00400000u)
                          : __builtin_bit_cast(float, uint32_t(min(sb, 254)) << 23);
  typedef short s2_t __attribute__((ext_vector_type(2)));
  typedef __bf16 bf2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  int hi[8], lo[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int sidx = fp4_src(FMT, 4 * w + b);  // 8u + e
      h[b] = (sidx & 1) ? (v[sidx / 2] >> 16) : (v[sidx / 2] & 0xFFFFu);
    }
    s2_t ph = {0, 0}, pl = {0, 0};
    ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(ph, __builtin_bit_cast(bf2_t, h[0] | (h[1] << 16)), S, false);
    ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_bf16(ph, __builtin_bit_cast(bf2_t, h[2] | (h[3] << 16)), S, true);
    hi[w] = __builtin_bit_cast(int, ph);
    const f2_t b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[w], S, false);
    const f2_t b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[w], S, true);
    const float r0 = __builtin_bit_cast(float, h[0] << 16) - b01.x;
    const float r1 = __builtin_bit_cast(float, h[1] << 16) - b01.y;
    const float r2 = __builtin_bit_cast(float, h[2] << 16) - b23.x;
    const float r3 = __builtin_bit_cast(float, h[3] << 16) - b23.y;
    pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, r0, r1, S, false);
    pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, r2, r3, S, true);
    lo[w] = __builtin_bit_cast(int, pl);
  }
  o.h0 = u4_t{uint32_t(hi[0]), uint32_t(hi[1]), uint32_t(hi[2]), uint32_t(hi[3])};
  o.h1 = u4_t{uint32_t(hi[4]), uint32_t(hi[5]), uint32_t(hi[6]), uint32_t(hi[7])};
  o.l0 = u4_t{uint32_t(lo[0]), uint32_t(lo[1]), uint32_t(lo[2]), uint32_t(lo[3])};
  o.l1 = u4_t{uint32_t(lo[4]), uint32_t(lo[5]), uint32_t(lo[6]), uint32_t(lo[7])};
  o.sb = uint8_t(sb);
}

// fp16 x in three pieces: the same 32 values and nibble order, with pieces
// hi, mid and lo (x = S (hi + mid + lo)).  An fp16 value has 11 significant
// bits and each piece 4, so the split is exact for every value within 2^6
// of the block's largest (the lowest bit of those lands at or above 2^-9 of
// the scaled range, the smallest fp8 step); a value further below carries
// an error below 2^-17 of that largest, as in the two-piece bf16 split.  sb
// puts the largest magnitude in [128, 256) for normal values and scales
// fp16 subnormals as if their exponent were the smallest normal one (they
// then scale to at most 128 and stay exact); a block holding inf or nan
// gets the nan scale 0xFF.
struct XQuarter3 {
  u4_t h0, h1, m0, m1, l0, l1;
  uint8_t sb;
};

template <int FMT>
__device__ __forceinline__ void split_x_regs_f16(const u4_t (&x)[4], XQuarter3 &o) {
  uint32_t v[16];
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    v[4 * u + 0] = x[u].x;
    v[4 * u + 1] = x[u].y;
    v[4 * u + 2] = x[u].z;
    v[4 * u + 3] = x[u].w;
  }
  typedef unsigned short u2h_t __attribute__((ext_vector_type(2)));
  u2h_t m2 = {0, 0};
#pragma unroll
  for (int i = 0; i < 16; ++i) m2 = __builtin_elementwise_max(m2, __builtin_bit_cast(u2h_t, v[i] & 0x7FFF7FFFu));
  const uint32_t mx = max(uint32_t(m2.x), uint32_t(m2.y));
  const int ef = int(mx >> 10);  // fp16 exponent field of the largest magnitude
  const int sb = ef == 31 ? 255 : max(ef, 1) + 105;
  const float S = __builtin_bit_cast(float, uint32_t(min(sb, 254)) << 23);
  typedef short s2_t __attribute__((ext_vector_type(2)));
  typedef _Float16 h2_t __attribute__((ext_vector_type(2)));
  typedef float f2_t __attribute__((ext_vector_type(2)));
  int hi[8], mid[8], lo[8];
#pragma unroll
  for (int w = 0; w < 8; ++w) {
    uint32_t h[4];
#pragma unroll
    for (int b = 0; b < 4; ++b) {
      const int sidx = fp4_src(FMT, 4 * w + b);  // 8u + e
      h[b] = (sidx & 1) ? (v[sidx / 2] >> 16) : (v[sidx / 2] & 0xFFFFu);
    }
    s2_t ph = {0, 0}, pm = {0, 0}, pl = {0, 0};
    ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(ph, __builtin_bit_cast(h2_t, h[0] | (h[1] << 16)), S, false);
    ph = __builtin_amdgcn_cvt_scalef32_pk_fp8_f16(ph, __builtin_bit_cast(h2_t, h[2] | (h[3] << 16)), S, true);
    hi[w] = __builtin_bit_cast(int, ph);
    const f2_t b01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[w], S, false);
    const f2_t b23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(hi[w], S, true);
    // Residuals in fp32 are exact: both terms are multiples of the value's
    // lowest bit and the difference is below 2^4 of S.
    const float r0 = float(__builtin_bit_cast(_Float16, uint16_t(h[0]))) - b01.x;
    const float r1 = float(__builtin_bit_cast(_Float16, uint16_t(h[1]))) - b01.y;
    const float r2 = float(__builtin_bit_cast(_Float16, uint16_t(h[2]))) - b23.x;
    const float r3 = float(__builtin_bit_cast(_Float16, uint16_t(h[3]))) - b23.y;
    pm = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pm, r0, r1, S, false);
    pm = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pm, r2, r3, S, true);
    mid[w] = __builtin_bit_cast(int, pm);
    const f2_t c01 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(mid[w], S, false);
    const f2_t c23 = __builtin_amdgcn_cvt_scalef32_pk_f32_fp8(mid[w], S, true);
    pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, r0 - c01.x, r1 - c01.y, S, false);
    pl = __builtin_amdgcn_cvt_scalef32_pk_fp8_f32(pl, r2 - c23.x, r3 - c23.y, S, true);
    lo[w] = __builtin_bit_cast(int, pl);
  }
  o.h0 = u4_t{uint32_t(hi[0]), uint32_t(hi[1]), uint32_t(hi[2]), uint32_t(hi[3])};
  o.h1 = u4_t{uint32_t(hi[4]), uint32_t(hi[5]), uint32_t(hi[6]), uint32_t(hi[7])};
  o.m0 = u4_t{uint32_t(mid[0]), uint32_t(mid[1]), uint32_t(mid[2]), uint32_t(mid[3])};
  o.m1 = u4_t{uint32_t(mid[4]), uint32_t(mid[5]), uint32_t(mid[6]), uint32_t(mid[7])};
  o.l0 = u4_t{uint32_t(lo[0]), uint32_t(lo[1]), uint32_t(lo[2]), uint32_t(lo[3])};
  o.l1 = u4_t{uint32_t(lo[4]), uint32_t(lo[5]), uint32_t(lo[6]), uint32_t(lo[7])};
  o.sb = uint8_t(sb);
}

// The same from memory: src points at x[m][128 g + 8 q]; in == false gives
// zeros (src must still be a readable address).
template <int FMT>
__device__ __forceinline__ void split_x_quarter(const uint16_t *src, bool in, XQuarter &o) {
  u4_t x[4];
  const u4_t z = {0u, 0u, 0u, 0u};
#pragma unroll
  for (int u = 0; u < 4; ++u) {
    const u4_t v = *reinterpret_cast<const u4_t *>(src + 32 * u);
    x[u] = in ? v : z;
  }
  split_x_regs<FMT>(x, o);
}

// Workgroup barrier for data exchanged through LDS only: this wave's LDS
// operations complete (lgkmcnt), then s_barrier.  __syncthreads() would also
// wait for every global load in flight (its workgroup-scope fence includes
// vmcnt(0)), draining the weight prefetch at every pass or tile set.  The
// memory clobber keeps the compiler from moving any access across it.
__device__ __forceinline__ void lds_barrier() {
  asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
}

__device__ __forceinline__ float half_to_float(uint16_t h) {
  return float(__builtin_bit_cast(_Float16, h));
}

__device__ __forceinline__ float x_to_float(uint16_t v, bool bf) {
  return bf ? __builtin_bit_cast(float, uint32_t(v) << 16) : half_to_float(v);
}

__device__ __forceinline__ uint16_t float_to_half_rne(float f) {
  return __builtin_bit_cast(uint16_t, static_cast<_Float16>(f));
}

// Round-robin 1-D block ids over the 8 XCDs onto a tile order in which each
// XCD gets a contiguous run of tiles (tiles that share operand rows then
// share that XCD's L2).
__device__ __forceinline__ int xcd_swizzle(int bid, int nblocks) {
  const int per = nblocks / 8, rem = nblocks % 8;
  const int x = bid % 8, local = bid / 8;
  // XCD x runs blocks x, x+8, ... (per + (x < rem) of them): give it tiles
  // [x*per + min(x, rem), +count).
  return x * per + (x < rem ? x : rem) + local;
}

}  // namespace lowbit
