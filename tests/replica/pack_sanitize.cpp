// Sanitizer driver for the host packer (test infrastructure).
//
// Links the library's own pack.cpp (host code only) and calls its C ABI on
// buffers of exactly the sizes the ABI promises to touch, so that a build
// with AddressSanitizer + UBSan (or ThreadSanitizer, for the packer's worker
// threads) reports any out-of-bounds access, undefined arithmetic or data
// race.  Codes and scales come from a fixed-seed generator; every pack is
// unpacked again and compared with its input, and the error paths are
// called with too-small buffers and out-of-set codes.  Prints "ok" or the
// first mismatch and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <vector>

#include "../../include/lowbit.h"

namespace {

uint64_t rng_state = 0x9E3779B97F4A7C15ull;
uint64_t next_u64() {  // splitmix64
  uint64_t z = (rng_state += 0x9E3779B97F4A7C15ull);
  z = (z ^ (z >> 30)) * 0xBF58476D1CE4E5B9ull;
  z = (z ^ (z >> 27)) * 0x94D049BB133111EBull;
  return z ^ (z >> 31);
}

[[noreturn]] void fail(const char *what, int fmt, long long N, long long K) {
  std::printf("FAIL %s fmt=%d N=%lld K=%lld\n", what, fmt, N, K);
  std::exit(1);
}

// Exact-size heap buffer (ASan traps one byte past the end).
template <class T>
T *alloc(int64_t n) {
  return static_cast<T *>(std::malloc(size_t(n > 0 ? n : 1) * sizeof(T)));
}

void round_trip(int fmt, int64_t N, int64_t K) {
  const int64_t G = K / 128;
  int8_t *codes = alloc<int8_t>(N * K);
  uint16_t *sc = alloc<uint16_t>(N * G);
  for (int64_t i = 0; i < N * K; ++i) {
    const uint64_t r = next_u64() % 3;
    codes[i] = fmt == LOWBIT_Q1_G128 ? (r & 1 ? 1 : -1) : int8_t(int(r) - 1);
  }
  for (int64_t i = 0; i < N * G; ++i) sc[i] = uint16_t(next_u64());
  const int64_t bytes = packed_bytes_lowbit(fmt, N, K);
  if (bytes < 0) fail("packed_bytes", fmt, N, K);
  uint8_t *blob = alloc<uint8_t>(bytes);
  const int st = fmt == LOWBIT_Q1_G128 ? pack_q1_g128(codes, sc, N, K, blob, bytes)
                 : fmt == LOWBIT_TQ2_G128 ? pack_tq2_g128(codes, sc, N, K, blob, bytes)
                                          : pack_tq5_g128(codes, sc, N, K, blob, bytes);
  if (st != LOWBIT_OK) fail("pack", fmt, N, K);
  int8_t *c2 = alloc<int8_t>(N * K);
  uint16_t *s2 = alloc<uint16_t>(N * G);
  if (unpack_lowbit(fmt, blob, bytes, N, K, c2, s2) != LOWBIT_OK) fail("unpack", fmt, N, K);
  if (N * K && std::memcmp(codes, c2, size_t(N * K))) fail("codes round trip", fmt, N, K);
  if (N * G && std::memcmp(sc, s2, size_t(N * G) * 2)) fail("scales round trip", fmt, N, K);
  // Codes only, scales only.
  if (unpack_lowbit(fmt, blob, bytes, N, K, c2, nullptr) != LOWBIT_OK) fail("unpack codes", fmt, N, K);
  if (unpack_lowbit(fmt, blob, bytes, N, K, nullptr, s2) != LOWBIT_OK) fail("unpack scales", fmt, N, K);
  // Error paths: a blob one byte short, an out-of-set code.
  if (bytes > 0) {
    if (unpack_lowbit(fmt, blob, bytes - 1, N, K, c2, s2) != LOWBIT_ERR_SIZE) fail("short blob", fmt, N, K);
    const int short_st = fmt == LOWBIT_Q1_G128 ? pack_q1_g128(codes, sc, N, K, blob, bytes - 1)
                         : fmt == LOWBIT_TQ2_G128 ? pack_tq2_g128(codes, sc, N, K, blob, bytes - 1)
                                                  : pack_tq5_g128(codes, sc, N, K, blob, bytes - 1);
    if (short_st != LOWBIT_ERR_SIZE) fail("short out", fmt, N, K);
    codes[N * K - 1] = fmt == LOWBIT_Q1_G128 ? 0 : 2;
    const int bad = fmt == LOWBIT_Q1_G128 ? pack_q1_g128(codes, sc, N, K, blob, bytes)
                    : fmt == LOWBIT_TQ2_G128 ? pack_tq2_g128(codes, sc, N, K, blob, bytes)
                                             : pack_tq5_g128(codes, sc, N, K, blob, bytes);
    if (bad != LOWBIT_ERR_VALUE) fail("out-of-set code", fmt, N, K);
  }
  std::free(codes);
  std::free(sc);
  std::free(blob);
  std::free(c2);
  std::free(s2);
}

void mlx_import(int64_t N, int64_t K, int dtype) {
  const int64_t G = K / 128, esz = dtype == LOWBIT_F32 ? 4 : 2;
  uint32_t *wq = alloc<uint32_t>(N * K / 32);
  for (int64_t i = 0; i < N * K / 32; ++i) wq[i] = uint32_t(next_u64());
  uint8_t *a = alloc<uint8_t>(N * G * esz), *b = alloc<uint8_t>(N * G * esz);
  for (int64_t i = 0; i < N * G; ++i) {
    // scale a = 2 s, bias b = -s with s = 2^-6 (exact in every dtype)
    if (dtype == LOWBIT_F32) {
      const float av = 0.03125f, bv = -0.015625f;
      std::memcpy(a + 4 * i, &av, 4);
      std::memcpy(b + 4 * i, &bv, 4);
    } else {
      const uint16_t av = dtype == LOWBIT_F16 ? 0x2800 : 0x3D00, bv = dtype == LOWBIT_F16 ? 0xA400 : 0xBC80;
      std::memcpy(a + 2 * i, &av, 2);
      std::memcpy(b + 2 * i, &bv, 2);
    }
  }
  const int64_t bytes = packed_bytes_lowbit(LOWBIT_Q1_G128, N, K);
  uint8_t *blob = alloc<uint8_t>(bytes);
  if (import_mlx_q1_g128(wq, a, b, dtype, N, K, blob, bytes) != LOWBIT_OK) fail("mlx import", 1, N, K);
  int8_t *c2 = alloc<int8_t>(N * K);
  uint16_t *s2 = alloc<uint16_t>(N * G);
  if (unpack_lowbit(LOWBIT_Q1_G128, blob, bytes, N, K, c2, s2) != LOWBIT_OK) fail("mlx unpack", 1, N, K);
  for (int64_t n = 0; n < N; ++n)
    for (int64_t k = 0; k < K; ++k) {
      const int q = int((wq[(n * K + k) / 32] >> (k % 32)) & 1);
      if (c2[n * K + k] != (q ? 1 : -1)) fail("mlx bits", 1, N, K);
    }
  for (int64_t i = 0; i < N * G; ++i)
    if (s2[i] != 0x2400) fail("mlx scale", 1, N, K);
  std::free(wq);
  std::free(a);
  std::free(b);
  std::free(blob);
  std::free(c2);
  std::free(s2);
}

}  // namespace

int main() {
  const int64_t shapes[][2] = {{1, 128}, {2, 256}, {15, 384}, {16, 512}, {17, 640}, {31, 768}, {33, 1152},
                               {16, 1280}, {5, 2048}, {40, 896}, {48, 17408}, {300, 5120}, {0, 128}, {3, 0}};
  for (int fmt = LOWBIT_Q1_G128; fmt <= LOWBIT_TQ5_G128; ++fmt)
    for (const auto &s : shapes) round_trip(fmt, s[0], s[1]);
  for (int dt = LOWBIT_F16; dt <= LOWBIT_F32; ++dt) mlx_import(37, 1408, dt);
  std::printf("ok\n");
  return 0;
}
