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
