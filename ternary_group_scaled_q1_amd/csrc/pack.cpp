// Host packer / unpacker: codes + FP16 scales <-> device layout v2 blob.
//
// Value maps: Binary g128 stores bit 1 for +scale and bit 0 for -scale
// (lnrk.cn page, Binary g128 section); Ternary g128 stores t in {-1,0,+1}
// either as the 2-bit code t + 1 (2-bit slots, ksqn.cn page) or as base-3
// digits t + 1, five per byte (cnblogs.com page, section 2.4).  The
// arrangement of bits and scales is the device layout v2 described in
// layout.hpp.
#include <algorithm>
#include <atomic>
#include <cmath>
#include <cstring>
#include <limits>
#include <thread>
#include <vector>

#include "../../include/lowbit.h"
#include "layout.hpp"

namespace lowbit {

// Run f(i) for i in [0, n) on up to hardware_concurrency() threads.
template <class F>
static void parallel_for(int64_t n, F f) {
  int64_t nt = std::max(1u, std::thread::hardware_concurrency());
  nt = std::min<int64_t>(nt, std::max<int64_t>(1, n / 4));
  if (nt <= 1) {
    for (int64_t i = 0; i < n; ++i) f(i);
    return;
  }
  std::atomic<int64_t> next(0);
  std::vector<std::thread> th;
  for (int64_t t = 0; t < nt; ++t)
    th.emplace_back([&]() {
      for (int64_t i; (i = next.fetch_add(1)) < n;) f(i);
    });
  for (auto &x : th) x.join();
}

static void store_u32(uint8_t *p, uint32_t w) {
  p[0] = uint8_t(w); p[1] = uint8_t(w >> 8); p[2] = uint8_t(w >> 16); p[3] = uint8_t(w >> 24);
}
static uint32_t load_u32(const uint8_t *p) {
  return uint32_t(p[0]) | uint32_t(p[1]) << 8 | uint32_t(p[2]) << 16 | uint32_t(p[3]) << 24;
}

static bool codes_valid(const int8_t *codes, int64_t n, bool binary) {
  std::atomic<bool> ok(true);
  int64_t blocks = (n + (1 << 20) - 1) >> 20;
  parallel_for(blocks, [&](int64_t b) {
    int64_t lo = b << 20, hi = std::min(n, lo + (int64_t(1) << 20));
    for (int64_t i = lo; i < hi; ++i) {
      int8_t c = codes[i];
      if (binary ? (c != 1 && c != -1) : (c < -1 || c > 1)) { ok = false; return; }
    }
  });
  return ok;
}

// ------------------------------------------------------------- q1 / tq2 ---
// code(n, k) gives the code of row n, column k (-1/+1, or -1/0/+1).
template <class Code>
static void pack_bits(int fmt, Code code, const Geom &g, uint8_t *plane) {
  const int64_t unit = fmt == 1 ? 16 : 32;
  parallel_for(g.tiles, [&](int64_t T) {
    const int64_t R = std::min<int64_t>(16, g.N - 16 * T);
    for (int64_t c = 0; c < g.chunks; ++c) {
      const int64_t Gc = std::min<int64_t>(4, g.G - 4 * c);
      uint8_t *blk = plane + chunk_offset(g, T, c, unit);
      for (int q = 0; q < 4; ++q)
        for (int64_t j = 0; j < R; ++j)
          for (int64_t gi = 0; gi < Gc; ++gi) {
            const int64_t n = 16 * T + j, k0 = (4 * c + gi) * kGroup;
            if (fmt == 1) {
              uint32_t w = 0;
              for (int u = 0; u < 4; ++u)
                for (int e = 0; e < 8; ++e)
                  if (code(n, k0 + 32 * u + 8 * q + e) == 1) w |= 1u << q1_pos(u, e);
              store_u32(blk + 4 * ((q * R + j) * Gc + gi), w);
            } else {
              const int64_t hh = gi / 2, Gh = std::min<int64_t>(2, Gc - 2 * hh);
              uint8_t *half = blk + R * 64 * hh;
              for (int v = 0; v < 2; ++v) {
                uint32_t w = 0;
                for (int uu = 0; uu < 2; ++uu)
                  for (int e = 0; e < 8; ++e) {
                    int u = 2 * v + uu;
                    const uint32_t cv = uint32_t(code(n, k0 + 32 * u + 8 * q + e) + 1);
                    w |= cv << tq2_pos(u, e);
                  }
                store_u32(half + 4 * (((q * R + j) * Gh + (gi - 2 * hh)) * 2 + v), w);
              }
            }
          }
    }
  });
}

static bool unpack_bits(int fmt, const uint8_t *plane, const Geom &g, int8_t *codes) {
  const int64_t unit = fmt == 1 ? 16 : 32;
  std::atomic<bool> ok(true);
  parallel_for(g.tiles, [&](int64_t T) {
    const int64_t R = std::min<int64_t>(16, g.N - 16 * T);
    for (int64_t c = 0; c < g.chunks; ++c) {
      const int64_t Gc = std::min<int64_t>(4, g.G - 4 * c);
      const uint8_t *blk = plane + chunk_offset(g, T, c, unit);
      for (int q = 0; q < 4; ++q)
        for (int64_t j = 0; j < R; ++j)
          for (int64_t gi = 0; gi < Gc; ++gi) {
            int8_t *row = codes ? codes + (16 * T + j) * g.K + (4 * c + gi) * kGroup : nullptr;
            if (fmt == 1) {
              uint32_t w = load_u32(blk + 4 * ((q * R + j) * Gc + gi));
              if (row)
                for (int u = 0; u < 4; ++u)
                  for (int e = 0; e < 8; ++e)
                    row[32 * u + 8 * q + e] = ((w >> q1_pos(u, e)) & 1) ? 1 : -1;
            } else {
              const int64_t hh = gi / 2, Gh = std::min<int64_t>(2, Gc - 2 * hh);
              const uint8_t *half = blk + R * 64 * hh;
              for (int v = 0; v < 2; ++v) {
                uint32_t w = load_u32(half + 4 * (((q * R + j) * Gh + (gi - 2 * hh)) * 2 + v));
                for (int uu = 0; uu < 2; ++uu)
                  for (int e = 0; e < 8; ++e) {
                    int u = 2 * v + uu;
                    uint32_t code = (w >> tq2_pos(u, e)) & 3;
                    if (code == 3) ok = false;
                    if (row) row[32 * u + 8 * q + e] = int8_t(int(code) - 1);
                  }
              }
            }
          }
    }
  });
  return ok;
}

// ------------------------------------------------------------------ tq5 ---
static const int kPow3[5] = {1, 3, 9, 27, 81};

static void pack_tq5(const int8_t *codes, const Geom &g, uint8_t *plane) {
  const Tq5Geom t = tq5_geom(g.K);
  parallel_for(g.tiles, [&](int64_t T) {
    const int64_t R = std::min<int64_t>(16, g.N - 16 * T);
    uint8_t *tile = plane + 16 * T * t.rowbytes;
    for (int64_t j = 0; j < R; ++j) {
      const int8_t *row = codes + (16 * T + j) * g.K;
      for (int64_t S = 0; S < t.s_full; ++S) {
        uint8_t *seg = tile + R * 128 * S;
        for (int b = 0; b < 128; ++b) {
          int v = 0;
          for (int i = 0; i < 5; ++i) v += (row[640 * S + 128 * i + b] + 1) * kPow3[i];
          int u = b >> 5, q = (b >> 3) & 3, e = b & 7, w = 8 * u + e;
          seg[R * 64 * (w >> 4) + (q * R + j) * 16 + (w & 15)] = uint8_t(v);
        }
      }
      uint8_t *tail = tile + R * 128 * t.s_full + j * t.b_tail;
      for (int64_t b = 0; b < t.b_tail; ++b) {
        int v = 0;
        for (int i = 0; i < 5; ++i) {
          int64_t ks = b + t.b_tail * i;
          int d = ks < t.L_tail ? row[640 * t.s_full + ks] + 1 : 1;
          v += d * kPow3[i];
        }
        tail[b] = uint8_t(v);
      }
    }
  });
}

static bool unpack_tq5(const uint8_t *plane, const Geom &g, int8_t *codes) {
  const Tq5Geom t = tq5_geom(g.K);
  std::atomic<bool> ok(true);
  parallel_for(g.tiles, [&](int64_t T) {
    const int64_t R = std::min<int64_t>(16, g.N - 16 * T);
    const uint8_t *tile = plane + 16 * T * t.rowbytes;
    for (int64_t j = 0; j < R; ++j) {
      int8_t *row = codes ? codes + (16 * T + j) * g.K : nullptr;
      for (int64_t S = 0; S < t.s_full; ++S) {
        const uint8_t *seg = tile + R * 128 * S;
        for (int b = 0; b < 128; ++b) {
          int u = b >> 5, q = (b >> 3) & 3, e = b & 7, w = 8 * u + e;
          int v = seg[R * 64 * (w >> 4) + (q * R + j) * 16 + (w & 15)];
          if (v >= 243) { ok = false; continue; }
          if (row)
            for (int i = 0; i < 5; ++i) row[640 * S + 128 * i + b] = int8_t((v / kPow3[i]) % 3 - 1);
        }
      }
      const uint8_t *tail = tile + R * 128 * t.s_full + j * t.b_tail;
      for (int64_t b = 0; b < t.b_tail; ++b) {
        int v = tail[b];
        if (v >= 243) { ok = false; continue; }
        for (int i = 0; i < 5; ++i) {
          int64_t ks = b + t.b_tail * i;
          int d = (v / kPow3[i]) % 3;
          if (ks < t.L_tail) {
            if (row) row[640 * t.s_full + ks] = int8_t(d - 1);
          } else if (d != 1) {
            ok = false;
          }
        }
      }
    }
  });
  return ok;
}

// Row-major scales [N][G] <-> plane B: row j's G_c scales of a chunk are
// contiguous on both sides.  Plane B may be only 2-byte aligned (tq5).
static void scatter_scales(int fmt, const Geom &g, const uint16_t *rows, uint8_t *pb) {
  const int W = scale_chunk_groups(fmt);
  parallel_for(g.N, [&](int64_t n) {
    for (int64_t c = 0; c * W < g.G; ++c) {
      const int64_t gc = std::min<int64_t>(W, g.G - W * c);
      std::memcpy(pb + 2 * scale_index(g.N, g.G, W, n, W * c), rows + n * g.G + W * c, size_t(2 * gc));
    }
  });
}

static void gather_scales(int fmt, const Geom &g, const uint8_t *pb, uint16_t *rows) {
  const int W = scale_chunk_groups(fmt);
  parallel_for(g.N, [&](int64_t n) {
    for (int64_t c = 0; c * W < g.G; ++c) {
      const int64_t gc = std::min<int64_t>(W, g.G - W * c);
      std::memcpy(rows + n * g.G + W * c, pb + 2 * scale_index(g.N, g.G, W, n, W * c), size_t(2 * gc));
    }
  });
}

static int check_fmt_shape(int fmt, int64_t N, int64_t K) {
  if (fmt < 1 || fmt > 3) return LOWBIT_ERR_ENUM;
  if (N < 0 || K < 0 || K % kGroup) return LOWBIT_ERR_SHAPE;
  return LOWBIT_OK;
}

static int pack_any(int fmt, const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K,
                    void *out, int64_t out_bytes) {
  int st = check_fmt_shape(fmt, N, K);
  if (st) return st;
  const int64_t need = packed_bytes_lowbit(fmt, N, K);
  if (need > 0 && (!codes || !scales || !out)) return LOWBIT_ERR_NULL;
  if (out_bytes < need) return LOWBIT_ERR_SIZE;
  if (need == 0) return LOWBIT_OK;
  if (!codes_valid(codes, N * K, fmt == 1)) return LOWBIT_ERR_VALUE;
  const Geom g = geom(N, K);
  uint8_t *plane = static_cast<uint8_t *>(out);
  if (fmt == 3) pack_tq5(codes, g, plane);
  else pack_bits(fmt, [&](int64_t n, int64_t k) { return codes[n * K + k]; }, g, plane);
  scatter_scales(fmt, g, scales, plane + plane_a_bytes(fmt, N, K));
  return LOWBIT_OK;
}

// ------------------------------------------------------------ MLX import ---
// MLX's grouped affine format stores, per group of 128 weights, a scale and
// a bias next to the packed bits, w = scale * q + bias, which is why its 1-bit
// package costs 1.25 bits per weight against 1.125 for the scale-only
// format (lnrk.cn page, MLX packing paragraph; aberweb.com page, summary
// section 2).  A group whose two values are {bias, scale + bias} = {-s, +s},
// i.e. scale = -2 bias, is a Binary g128 group with scale s = -bias and the
// same bits (bit 1 -> +s).

static double half_value(uint16_t h) {
  const int e = (h >> 10) & 31, f = h & 1023;
  double v;
  if (e == 31) v = f ? std::numeric_limits<double>::quiet_NaN() : std::numeric_limits<double>::infinity();
  else if (e == 0) v = std::ldexp(double(f), -24);
  else v = std::ldexp(double(1024 + f), e - 25);
  return (h & 0x8000) ? -v : v;
}

static double float_value(uint32_t u) {
  float f;
  std::memcpy(&f, &u, 4);
  return double(f);
}

// The FP16 pattern of v when v is exactly representable, else false.
static bool half_exact(double v, uint16_t &out) {
  if (!std::isfinite(v)) return false;
  const uint16_t sign = std::signbit(v) ? 0x8000 : 0;
  const double a = std::fabs(v);
  if (a == 0.0) { out = sign; return true; }
  if (a > 65504.0) return false;
  int E;
  std::frexp(a, &E);  // a = m 2^E, m in [0.5, 1)
  const int e = E - 1;
  if (e >= -14) {
    const double f = std::ldexp(a, 10 - e);  // in [1024, 2048)
    if (f != std::floor(f)) return false;
    out = uint16_t(sign | ((e + 15) << 10) | (uint16_t(f) - 1024));
  } else {
    const double f = std::ldexp(a, 24);
    if (f != std::floor(f)) return false;
    out = uint16_t(sign | uint16_t(f));
  }
  return true;
}

static double affine_value(const void *base, int dtype, int64_t i) {
  if (dtype == LOWBIT_F32) return float_value(static_cast<const uint32_t *>(base)[i]);
  const uint16_t h = static_cast<const uint16_t *>(base)[i];
  return dtype == LOWBIT_F16 ? half_value(h) : float_value(uint32_t(h) << 16);
}

}  // namespace lowbit

using namespace lowbit;

extern "C" {

int64_t packed_bytes_lowbit(int fmt, int64_t N, int64_t K) {
  int st = check_fmt_shape(fmt, N, K);
  if (st) return st;
  return plane_a_bytes(fmt, N, K) + N * (K / kGroup) * 2;
}

int pack_q1_g128(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K, void *out,
                 int64_t out_bytes) {
  return pack_any(1, codes, scales, N, K, out, out_bytes);
}
int pack_tq2_g128(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K, void *out,
                  int64_t out_bytes) {
  return pack_any(2, codes, scales, N, K, out, out_bytes);
}
int pack_tq5_g128(const int8_t *codes, const uint16_t *scales, int64_t N, int64_t K, void *out,
                  int64_t out_bytes) {
  return pack_any(3, codes, scales, N, K, out, out_bytes);
}

int import_mlx_q1_g128(const uint32_t *wq, const void *scales, const void *biases, int sb_dtype, int64_t N,
                       int64_t K, void *out, int64_t out_bytes) {
  if (sb_dtype < LOWBIT_F16 || sb_dtype > LOWBIT_F32) return LOWBIT_ERR_ENUM;
  int st = check_fmt_shape(1, N, K);
  if (st) return st;
  const int64_t need = packed_bytes_lowbit(1, N, K);
  if (need > 0 && (!wq || !scales || !biases || !out)) return LOWBIT_ERR_NULL;
  if (out_bytes < need) return LOWBIT_ERR_SIZE;
  if (need == 0) return LOWBIT_OK;
  const Geom g = geom(N, K);
  // Every group is checked before anything is written.
  std::vector<uint16_t> sc(size_t(N * g.G));
  std::atomic<bool> ok(true);
  parallel_for(N, [&](int64_t n) {
    for (int64_t gi = 0; gi < g.G; ++gi) {
      const double a = affine_value(scales, sb_dtype, n * g.G + gi);
      const double b = affine_value(biases, sb_dtype, n * g.G + gi);
      uint16_t h;
      if (!std::isfinite(a) || a != -2.0 * b || !half_exact(-b, h)) {
        ok = false;
        return;
      }
      sc[size_t(n * g.G + gi)] = h;
    }
  });
  if (!ok) return LOWBIT_ERR_VALUE;
  const int64_t words = K / 32;
  uint8_t *plane = static_cast<uint8_t *>(out);
  pack_bits(1, [&](int64_t n, int64_t k) -> int8_t { return ((wq[n * words + k / 32] >> (k % 32)) & 1) ? 1 : -1; },
            g, plane);
  scatter_scales(1, g, sc.data(), plane + plane_a_bytes(1, N, K));
  return LOWBIT_OK;
}

int unpack_lowbit(int fmt, const void *packed, int64_t packed_bytes, int64_t N, int64_t K,
                  int8_t *codes_out, uint16_t *scales_out) {
  int st = check_fmt_shape(fmt, N, K);
  if (st) return st;
  const int64_t need = packed_bytes_lowbit(fmt, N, K);
  if (need > 0 && !packed) return LOWBIT_ERR_NULL;
  if (packed_bytes < need) return LOWBIT_ERR_SIZE;
  if (need == 0) return LOWBIT_OK;
  const Geom g = geom(N, K);
  const uint8_t *plane = static_cast<const uint8_t *>(packed);
  // Validate first so that nothing is written on error.
  bool ok = fmt == 3 ? unpack_tq5(plane, g, nullptr) : unpack_bits(fmt, plane, g, nullptr);
  if (!ok) return LOWBIT_ERR_VALUE;
  if (codes_out) {
    if (fmt == 3) unpack_tq5(plane, g, codes_out);
    else unpack_bits(fmt, plane, g, codes_out);
  }
  if (scales_out) gather_scales(fmt, g, plane + plane_a_bytes(fmt, N, K), scales_out);
  return LOWBIT_OK;
}

}  // extern "C"
