// Decode GEMV with K-sliced waves, 9..16 tokens: Y[m][n] = sum_k X[m][k]
// t[n][k] s[n][k/128] (the group scale applied to exact products, as on the
// aberweb.com page, section 4.1: signs decoded inside the kernel, no dense
// weight tensor).
//
// A workgroup owns T row tiles and all of K; wave w owns chunk w of K (4
// groups, 512 weights), so a workgroup has K / 512 waves (8 or 10).  Each wave puts the
// A operands of its chunk (16 token rows x 512 k) into registers once, then
// walks the workgroup's T tiles: per tile one 1 KB (tq2: 2 KB) weight load
// per wave, decode, MFMAs, and the FP16 group scale on each fresh tile.  At
// every step the waves of a workgroup read the T-th tile's chunks, which lie
// next to each other (one contiguous run per tile in device layout v2).  The
// waves' sums of a tile meet once, in LDS, and are added in K order.
//
// Compared with the 2-D split kernel (x staged in LDS in passes, one wave
// per tile, K cut across workgroups for small matrices) there is no pass
// barrier, no LDS traffic for x and no sum across workgroups; every
// workgroup converts all of x, which pays off from three tiles per
// workgroup on.
//
// A operands:
//  * binary weights, bf16 x: fp8 pieces on the scaled 16x16x128 MFMA.  Lane
//    (q, r) converts quarter q of token r's group (split_x_regs: hardware k
//    32q .. 32q + 31, one E8M0 scale), and takes the halves its own k range
//    (16q .. 16q + 15 and 64 + 16q .. 64 + 16q + 15) needs from the lanes of
//    quarters q / 2 and 2 + q / 2 of the same token (ds_bpermute);
//  * ternary weights, or fp16 x: exact f16 / bf16 x on 16x16x32, lane (q, r)
//    holding x[r][128 g + 32 u + 8 q .. + 8] for k-step u, as loaded.
// Tokens past M take token 0's x as it is: an A row feeds only the same row
// of the result, and those rows are never stored (zeroing them would put a
// select right after every x load and serialise the loads).
#include "device.hpp"
#include "gemv_common.hpp"
#include "kernels.hpp"
#include "layout.hpp"

namespace lowbit {

namespace {

constexpr int kFp4 = 0, kBf16 = 1, kF16 = 2;
constexpr int kRing = 3;       // weight units in flight per wave

struct KsParams {
  MatSet ms;
  const uint16_t *X;  // [M][K]
  int M, K, G, tiles;
  int y_f16;
};

template <int FMT, int MODE, int T, int NW>
__global__ void __launch_bounds__(64 * NW, 1) gemv_kslice_kernel(KsParams p) {
  extern __shared__ __align__(16) char lds[];
  constexpr bool FP4 = MODE == kFp4;
  constexpr bool BF = MODE == kBf16;
  constexpr int nw = NW;
  const int wave = uni(threadIdx.x >> 6), lane = threadIdx.x & 63;
  const int qa = lane >> 4, r = lane & 15;
  const int t0 = uni(blockIdx.x * T);
  const int c = wave;  // this wave's chunk of K
  const bool tok = r < p.M;
  const uint16_t *xg = p.X + (int64_t)(tok ? r : 0) * p.K + 512 * c;

  // A operands of the chunk's 4 groups.
  u4_t ah0[4], ah1[4], al0[4], al1[4];  // fp8 pieces (FP4)
  int sa[4];
  u4_t ax[4][4];  // exact x cells [group][k-step] (not FP4)
  if constexpr (FP4) {
    const int src0 = 4 * (16 * (qa >> 1) + r), src1 = 4 * (16 * (2 + (qa >> 1)) + r);
    const bool odd = qa & 1;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      u4_t x[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) x[u] = *reinterpret_cast<const u4_t *>(xg + 128 * g + 8 * qa + 32 * u);
      XQuarter xq;
      split_x_regs<FMT>(x, xq);
      sa[g] = xq.sb;
      u4_t a0, a1, b0, b1, c0, c1, d0, d1;
#pragma unroll
      for (int e = 0; e < 4; ++e) {
        a0[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src0, int(xq.h0[e])));
        a1[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src0, int(xq.h1[e])));
        b0[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src1, int(xq.h0[e])));
        b1[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src1, int(xq.h1[e])));
        c0[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src0, int(xq.l0[e])));
        c1[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src0, int(xq.l1[e])));
        d0[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src1, int(xq.l0[e])));
        d1[e] = uint32_t(__builtin_amdgcn_ds_bpermute(src1, int(xq.l1[e])));
      }
      ah0[g] = odd ? a1 : a0;
      ah1[g] = odd ? b1 : b0;
      al0[g] = odd ? c1 : c0;
      al1[g] = odd ? d1 : d0;
    }
  } else {
#pragma unroll
    for (int g = 0; g < 4; ++g)
#pragma unroll
      for (int u = 0; u < 4; ++u) ax[g][u] = *reinterpret_cast<const u4_t *>(xg + 128 * g + 32 * u + 8 * qa);
  }

  // Weights: a ring of kRing units, one tile each, issued after x (issued
  // before it they timed slower on the binary launches); tiles past the
  // launch re-read the last tile (their sums are never stored).
  TileSet<1> ts;
  Unit<FMT, 1> ring[kRing];
  auto load = [&](Unit<FMT, 1> &u, int t) {
    resolve_tiles<FMT, 1>(p, ts, uni(min(t0 + t, p.tiles - 1)));
    load_full<FMT, 1>(ts, u, c);
  };
#pragma unroll
  for (int d = 0; d < kRing; ++d) load(ring[d], min(d, T - 1));
  float acc[T][4];
#pragma unroll
  for (int t = 0; t < T; ++t) {
    const Unit<FMT, 1> &u = ring[t % kRing];
#pragma unroll
    for (int e = 0; e < 4; ++e) acc[t][e] = 0.f;
#pragma unroll
    for (int g = 0; g < 4; ++g) {
      const float s = half_to_float(uint16_t(u.s[0][g >> 1] >> (16 * (g & 1))));
      f4_t d;
      if constexpr (FP4) {
        const u4_t b = q1_fp4(u.w[0][g]);
        d = mfma_f8f4_acc(al0[g], al1[g], b, sa[g], mfma_f8f4(ah0[g], ah1[g], b, sa[g]));
      } else {
#pragma unroll
        for (int uu = 0; uu < 4; ++uu) {
          u4_t b;
          if constexpr (FMT == 1) b = q1_operand_pm1<BF>(u.w[0][g], uu);
          else b = tq2_operand(u.w[0][2 * g + (uu >> 1)], uu);
          d = uu == 0 ? mfma16x16x32_zero<BF>(ax[g][uu], b) : mfma16x16x32<BF>(ax[g][uu], b, d);
        }
      }
#pragma unroll
      for (int e = 0; e < 4; ++e) acc[t][e] = fmaf(s, d[e], acc[t][e]);
    }
    // The loop is unrolled (T is a compile-time count), so every path
    // issues the same loads and the wait before a tile's MFMAs covers that
    // tile only.
    if (t + kRing < T) load(ring[t % kRing], t + kRing);
  }

  // The waves' sums, [tile][wave][lane][4] in LDS, added in K order.
  float *red = reinterpret_cast<float *>(lds);
#pragma unroll
  for (int t = 0; t < T; ++t)
    *reinterpret_cast<f4_t *>(red + ((t * nw + wave) * 64 + lane) * 4) = f4_t{acc[t][0], acc[t][1], acc[t][2], acc[t][3]};
  lds_barrier();
  const float mul = FMT == 1 ? 1.f : 0.5f;  // ternary operands carry 2t
  for (int o = threadIdx.x; o < T * 256; o += 64 * nw) {
    const int t = o >> 8, ln = (o >> 2) & 63, e = o & 3;
    const int m = 4 * (ln >> 4) + e;
    if (t0 + t >= p.tiles || m >= p.M) continue;
    float v = 0.f;
    for (int w = 0; w < nw; ++w) v += red[((t * nw + w) * 64 + ln) * 4 + e];
    store_y(tile_ref(p.ms, t0 + t), ln & 15, m, v * mul, p.y_f16);
  }
}

// Tiles per workgroup the kernel is built for; the launch takes the fewest
// that keep the grid within one workgroup per CU.
constexpr int kTs[] = {4, 6, 9, 12};

template <int FMT, int MODE, int NW>
hipError_t launch_nw(const LaunchArgs &a, const KsParams &p, int T) {
  const dim3 grid((p.tiles + T - 1) / T), block(64 * NW);
  const int lds = T * NW * 1024;
  if (T == 4) hipLaunchKernelGGL((gemv_kslice_kernel<FMT, MODE, 4, NW>), grid, block, lds, a.stream, p);
  else if (T == 6) hipLaunchKernelGGL((gemv_kslice_kernel<FMT, MODE, 6, NW>), grid, block, lds, a.stream, p);
  else if (T == 9) hipLaunchKernelGGL((gemv_kslice_kernel<FMT, MODE, 9, NW>), grid, block, lds, a.stream, p);
  else hipLaunchKernelGGL((gemv_kslice_kernel<FMT, MODE, 12, NW>), grid, block, lds, a.stream, p);
  return hipGetLastError();
}

template <int FMT, int MODE>
hipError_t launch_mode(const LaunchArgs &a, const KsParams &p, int T, int nw) {
  return nw == 10 ? launch_nw<FMT, MODE, 10>(a, p, T) : launch_nw<FMT, MODE, 8>(a, p, T);
}

}  // namespace

bool launch_gemv_kslice(const LaunchArgs &a, hipError_t &err) {
  // 9..16 tokens, K of 8 or 10 whole chunks (4096 or 5120: the wave count is
  // a compile-time constant of the kernel), whole row tiles, and enough
  // tiles for three or more per workgroup at one workgroup per CU.
  if (a.M <= 8 || a.M > 16 || a.fmt == 3 || a.K % 512 != 0) return false;
  const int chunks = int(a.K / 512);
  if (chunks != 8 && chunks != 10) return false;
  for (int i = 0; i < a.nmat; ++i)
    if (a.Ns[i] % 16 != 0) return false;
  const int cus = num_cus();
  const int64_t tiles = (a.N + 15) / 16;
  if (tiles < 3LL * cus) return false;
  int T = 0;
  for (int t : kTs)
    if (!T && (tiles + t - 1) / t <= cus) T = t;
  if (!T) return false;
  const int mode = a.fmt == 1 ? (a.x_bf16 ? kFp4 : kF16) : (a.x_bf16 ? kBf16 : kF16);
  KsParams p{};
  p.ms = mat_set(a);
  p.X = a.X;
  p.M = int(a.M); p.K = int(a.K); p.G = int(a.K / kGroup);
  p.tiles = int(tiles);
  p.y_f16 = a.y_f16;
  if (a.plan) {
    lowbit_plan &o = plan_record(a, LOWBIT_KERNEL_GEMV_KSLICE, int((tiles + T - 1) / T), 64 * chunks, T * chunks * 1024);
    o.token_slots = 16;
    o.operands = mode == kFp4 ? LOWBIT_OPERANDS_FP8_FP4 : (mode == kBf16 ? LOWBIT_OPERANDS_BF16 : LOWBIT_OPERANDS_F16);
    o.whole_tiles = 1;
    o.tiles_per_wave = T;
    o.waves = chunks;
    o.k_ranges = 1;
    o.groups_per_range = int(a.K / kGroup);
    o.groups_per_pass = 4;
    o.ring = kRing;
    err = hipSuccess;
    return true;
  }
  if (a.fmt == 1) err = mode == kFp4 ? launch_mode<1, kFp4>(a, p, T, chunks) : launch_mode<1, kF16>(a, p, T, chunks);
  else err = mode == kBf16 ? launch_mode<2, kBf16>(a, p, T, chunks) : launch_mode<2, kF16>(a, p, T, chunks);
  return true;
}

}  // namespace lowbit
