// Device layout v2 geometry, shared by the host packer and the HIP kernels.
//
// Plane A is cut into row tiles of 16 rows (R_T = min(16, N - 16T) rows in
// tile T) and, inside a tile, into chunks of 4 groups of 128 weights
// (G_c = min(4, G - 4c) groups in chunk c).  Inside a group, the weight at
// offset kk (0..127) is named by
//     u = kk / 32  (MFMA k-step, 32 weights each),
//     q = (kk / 8) % 4  (the lane quad that feeds it to the matrix core),
//     e = kk % 8  (its slot among the quad's 8 operand halves).
// One lane (q, j) of a wave reads, per chunk, one 32-bit word per group (q1)
// or two (tq2) holding every weight of row 16T+j, group 4c+g with that q, so
// a full chunk of a full tile is one contiguous 1 KB wave load per 16 bytes
// per lane.  Bit positions are chosen so that one shift brings two weights to
// the f16/bf16 sign (bit 15/31) and exponent-MSB (bit 14/30) positions.
#pragma once
#include <stdint.h>

namespace lowbit {

constexpr int kGroup = 128;
constexpr int kTileRows = 16;
constexpr int kChunkGroups = 4;

struct Geom {
  int64_t N, K, G;       // rows, columns, groups per row
  int64_t tiles, chunks; // row tiles, group chunks
};

inline Geom geom(int64_t N, int64_t K) {
  Geom g;
  g.N = N; g.K = K; g.G = K / kGroup;
  g.tiles = (N + kTileRows - 1) / kTileRows;
  g.chunks = (g.G + kChunkGroups - 1) / kChunkGroups;
  return g;
}

// q1: bit of weight (u, e) inside its lane word.
inline int q1_pos(int u, int e) {
  return 16 * (e & 1) + 15 - ((e >> 1) & 1) - 2 * (2 * u + (e >> 2));
}
// tq2: low bit of the 2-bit code of weight (u, e) inside word u/2 of its lane pair.
inline int tq2_pos(int u, int e) {
  return 16 * (e & 1) + 14 - 2 * (4 * (u & 1) + (e >> 1));
}

// Byte offset of chunk c of tile T in plane A; unit = bytes per (row, group).
inline int64_t chunk_offset(const Geom &g, int64_t T, int64_t c, int64_t unit) {
  int64_t R = g.N - 16 * T < 16 ? g.N - 16 * T : 16;
  return 16 * T * g.G * unit + R * 4 * c * unit;
}

// tq5 geometry: 640-trit segments (5 groups) + a tail of K mod 640 trits.
struct Tq5Geom {
  int64_t s_full, L_tail, b_tail, rowbytes;
};
inline Tq5Geom tq5_geom(int64_t K) {
  Tq5Geom t;
  t.s_full = K / 640;
  t.L_tail = K - 640 * t.s_full;
  t.b_tail = (t.L_tail + 4) / 5;
  t.rowbytes = 128 * t.s_full + t.b_tail;
  return t;
}

inline int64_t plane_a_bytes(int fmt, int64_t N, int64_t K) {
  if (fmt == 1) return N * K / 8;
  if (fmt == 2) return N * K / 4;
  return N * ((K + 4) / 5);
}

// Plane B, the FP16 scales after plane A, in the order of the units that read
// them: tile T holds its R_T*G scales from index 16*T*G on; inside it the
// groups are cut into chunks of W (4 for q1 / tq2: plane A's chunks; 5 for
// tq5: its 640-trit segments), chunk c (G_c = min(W, G - W c) groups) starts
// at R_T*W*c and holds row j's G_c scales at j*G_c.  The 16 rows x W scales
// of a full unit are then one contiguous run of 16*W values.
__host__ __device__ constexpr int scale_chunk_groups(int fmt) { return fmt == 3 ? 5 : 4; }

__host__ __device__ inline int64_t scale_index(int64_t N, int64_t G, int W, int64_t n, int64_t g) {
  const int64_t T = n / 16, j = n % 16, c = g / W;
  const int64_t R = N - 16 * T < 16 ? N - 16 * T : 16;
  const int64_t Gc = G - W * c < W ? G - W * c : W;
  return 16 * T * G + R * W * c + j * Gc + (g - W * c);
}

}  // namespace lowbit
