// Bounds-checked host replica of the address arithmetic of the library's
// HIP kernels (test infrastructure; it shares no code with the library).
//
// For one product launch, given its shapes and the plan the library's own
// planner chose (lowbit_gemv_plan / lowbit_gemm_plan), this program walks
// every workgroup, wave and lane through the kernel's loop structure and
// forms every global-memory and LDS address the kernel forms: x, the packed
// weight planes, the FP16 scales, the workspace (partial sums and arrival
// counters), the outputs and the dynamic LDS.  Each access is checked
// against a buffer of exactly the size the caller hands the kernel, and the
// buffers are real host allocations, so a build with AddressSanitizer also
// traps any slip in this replica itself.  It further checks that
//   * every output element is written exactly once, by its final store;
//   * LDS reads of staged activations see the pass they belong to (double
//     buffering), and workspace partial sums are written before they are
//     summed;
//   * every arrival counter is back at zero when the launch ends.
//
// Usage: kernel_addressing key=value ...   (keys: see main()); prints "ok"
// or the first violation and exits 1.
#include <cstdint>
#include <cstdio>
#include <cstdlib>
#include <cstring>
#include <map>
#include <string>
#include <vector>

namespace {

[[noreturn]] void fail(const char *what, const std::string &detail) {
  std::printf("FAIL %s: %s\n", what, detail.c_str());
  std::fflush(stdout);
  std::exit(1);
}

std::string fmtv(const char *f, long long a, long long b = 0, long long c = 0, long long d = 0) {
  char buf[256];
  std::snprintf(buf, sizeof buf, f, a, b, c, d);
  return buf;
}

// A buffer of exactly n bytes with a per-byte shadow tag (the pass or
// writer that last wrote it; -1 = never written).
struct Buf {
  std::string name;
  int64_t n = 0;
  uint8_t *p = nullptr;
  std::vector<int16_t> tag;  // only kept where data flow is checked
  bool track = false;
  volatile uint64_t sink = 0;
  Buf(const std::string &nm, int64_t bytes, bool tr = false) : name(nm), n(bytes), track(tr) {
    p = static_cast<uint8_t *>(std::malloc(size_t(bytes > 0 ? bytes : 1)));
    std::memset(p, 0, size_t(bytes > 0 ? bytes : 1));
    if (track) tag.assign(size_t(bytes > 0 ? bytes : 1), int16_t(-1));
  }
  ~Buf() { std::free(p); }
  Buf(const Buf &) = delete;
  Buf &operator=(const Buf &) = delete;
  void check(int64_t off, int64_t bytes, const char *what) {
    if (off < 0 || bytes < 0 || off + bytes > n)
      fail(what, name + fmtv(": bytes [%lld, %lld) outside [0, %lld)", off, off + bytes, n));
  }
  // A load of bytes [off, off + bytes): range-checked, and its first and
  // last byte touched so that AddressSanitizer sees the access too.
  void read(int64_t off, int64_t bytes, const char *what) {
    check(off, bytes, what);
    if (bytes > 0) sink = sink + p[off] + p[off + bytes - 1];
  }
  // A read whose bytes must carry tag `want` (data written for this use).
  void read_tagged(int64_t off, int64_t bytes, int32_t want, const char *what) {
    read(off, bytes, what);
    if (!track) return;
    for (int64_t i = 0; i < bytes; ++i)
      if (tag[size_t(off + i)] != int16_t(want))
        fail(what, name + fmtv(": byte %lld holds tag %lld, expected %lld", off + i, tag[size_t(off + i)], want));
  }
  void write(int64_t off, int64_t bytes, const char *what, int32_t t = 0) {
    check(off, bytes, what);
    if (bytes > 0) {
      p[off] = uint8_t(p[off] + 1);
      p[off + bytes - 1] = uint8_t(p[off + bytes - 1] + 1);
    }
    if (track)
      for (int64_t i = 0; i < bytes; ++i) tag[size_t(off + i)] = int16_t(t);
  }
  uint32_t u32(int64_t off) {
    check(off, 4, "counter");
    uint32_t v;
    std::memcpy(&v, p + off, 4);
    return v;
  }
  void set_u32(int64_t off, uint32_t v) {
    check(off, 4, "counter");
    std::memcpy(p + off, &v, 4);
  }
};

int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

struct Mats {
  int fmt = 1;
  int nmat = 1;
  int64_t N[4] = {0, 0, 0, 0};
  int64_t K = 0, G = 0, M = 0;
  int ysz = 4;
  std::vector<Buf *> W, Y;
  std::vector<std::vector<int32_t>> ycount;  // final stores per output element
  int64_t tile_end[4] = {0, 0, 0, 0};
  int64_t tiles = 0;

  static int64_t plane_a(int fmt, int64_t N, int64_t K) {
    return fmt == 1 ? N * K / 8 : fmt == 2 ? N * K / 4 : N * ((K + 4) / 5);
  }
  int64_t sc_off(int i) const { return plane_a(fmt, N[i], K); }

  void init() {
    G = K / 128;
    int64_t e = 0;
    for (int i = 0; i < nmat; ++i) {
      e += cdiv(N[i], 16);
      tile_end[i] = e;
      W.push_back(new Buf("W" + std::to_string(i), plane_a(fmt, N[i], K) + N[i] * G * 2));
      Y.push_back(new Buf("Y" + std::to_string(i), M * N[i] * ysz));
      ycount.emplace_back(size_t(M * N[i]), 0);
    }
    tiles = e;
  }
  ~Mats() {
    for (auto *b : W) delete b;
    for (auto *b : Y) delete b;
  }
  // Matrix and local tile of launch tile vt (vt < tiles).
  void tile_ref(int64_t vt, int &mi, int64_t &t) const {
    if (vt < 0 || vt >= tiles) fail("tile_ref", fmtv("tile %lld of %lld", vt, tiles));
    mi = 0;
    int64_t start = 0;
    while (vt >= tile_end[mi]) start = tile_end[mi++];
    t = vt - start;
  }
  int64_t rows_of(int mi, int64_t t) const { return N[mi] - 16 * t < 16 ? N[mi] - 16 * t : 16; }
  // store_y: row 16 t + j of matrix mi, token m (rows past N are skipped).
  void store_y(int mi, int64_t t, int64_t j, int64_t m) {
    const int64_t n = 16 * t + j;
    if (n >= N[mi]) return;
    if (m < 0 || m >= M) fail("store_y", fmtv("token %lld of %lld", m, M));
    Y[mi]->write((m * N[mi] + n) * ysz, ysz, "store_y");
    ++ycount[mi][size_t(m * N[mi] + n)];
  }
  void check_outputs() const {
    for (int i = 0; i < nmat; ++i)
      for (int64_t x = 0; x < M * N[i]; ++x)
        if (ycount[i][size_t(x)] != 1)
          fail("outputs", fmtv("matrix %lld element (m=%lld, n=%lld) stored %lld times", i, x / N[i], x % N[i],
                               ycount[i][size_t(x)]));
  }
};

// ------------------------------------------------ packed weight units ----
// load_unit (general path) of gemv_common.hpp: R tiles from t0, chunk c.
void load_unit(Mats &ms, int fmt, int R, int64_t t0, int64_t c, bool valid) {
  const int64_t unit = fmt == 1 ? 16 : 32;
  if (!valid) { c = 0; t0 = 0; }
  const int64_t Gc = std::min<int64_t>(4, ms.G - 4 * c);
  if (Gc <= 0) fail("load_unit", fmtv("chunk %lld of %lld groups", c, ms.G));
  for (int r = 0; r < R; ++r) {
    int mi;
    int64_t t;
    ms.tile_ref(std::min<int64_t>(t0 + r, ms.tiles - 1), mi, t);
    Buf &W = *ms.W[mi];
    const int64_t RT = ms.rows_of(mi, t);
    const int64_t blk = 16 * t * ms.G * unit + RT * 4 * c * unit;
    const int64_t sblk = ms.sc_off(mi) + 2 * (16 * t * ms.G + RT * 4 * c);
    for (int lane = 0; lane < 64; ++lane) {
      const int j = lane & 15, q = lane >> 4;
      if (RT == 16 && Gc == 4) {
        W.read(blk + 16 * lane, 16, "weights (whole unit)");
        if (fmt == 2) W.read(blk + 1024 + 16 * lane, 16, "weights (whole unit)");
        W.read(sblk + 2 * 4 * j, 8, "scales (whole unit)");
      } else {
        const int64_t jj = std::min<int64_t>(j, RT - 1);
        for (int g = 0; g < 4; ++g) {
          const int64_t gg = std::min<int64_t>(g, Gc - 1);
          if (fmt == 1) {
            W.read(blk + 4 * ((q * RT + jj) * Gc + gg), 4, "weights (ragged unit)");
          } else {
            const int64_t hh = gg >> 1, Gh = std::min<int64_t>(2, Gc - 2 * hh);
            W.read(blk + 4 * (RT * 16 * hh + ((q * RT + jj) * Gh + (gg - 2 * hh)) * 2), 8, "weights (ragged unit)");
          }
          W.read(sblk + 2 * (jj * Gc + gg), 2, "scales (ragged unit)");
        }
      }
    }
  }
}

// resolve_tiles + load_full: whole tiles, chunk c.
void load_full(Mats &ms, int fmt, int R, int64_t t0, int64_t c) {
  const int64_t unit = fmt == 1 ? 16 : 32, cb = fmt == 1 ? 1024 : 2048;
  for (int r = 0; r < R; ++r) {
    int mi;
    int64_t t;
    ms.tile_ref(std::min<int64_t>(t0 + r, ms.tiles - 1), mi, t);
    Buf &W = *ms.W[mi];
    for (int lane = 0; lane < 64; ++lane) {
      const int j = lane & 15;
      const int64_t w = 16 * t * ms.G * unit + c * cb + 16 * lane;
      W.read(w, 16, "weights (whole tiles)");
      if (fmt == 2) W.read(w + 1024, 16, "weights (whole tiles)");
      W.read(ms.sc_off(mi) + 2 * (16 * t * ms.G + 4 * j + 64 * c), 8, "scales (whole tiles)");
    }
  }
}

// --------------------------------------------------------- split kernel ----
void split_kernel(Mats &ms, std::map<std::string, int64_t> &P, Buf &X, Buf &ws) {
  const int fmt = ms.fmt;
  const int NW = int(P["waves"]), R = int(P["tiles_per_wave"]), KS = int(P["k_ranges"]);
  const int GK = int(P["groups_per_range"]), GP = int(P["groups_per_pass"]), MP = int(P["token_slots"]);
  const int ops = int(P["operands"]);
  const bool fp4 = ops == 3, full = P["whole_tiles"] != 0;
  const int64_t G = ms.G, M = ms.M, K = ms.K;
  const int64_t NV = 16 * ms.tiles;
  const int64_t row_blocks = cdiv(ms.tiles, NW * R);
  const int kRowBytes = 144;
  const int64_t buf_bytes = fp4 ? (GP * 2 * MP * kRowBytes + GP * MP * 4 + 15) / 16 * 16 : GP * 16 * MP * 16 + 16;
  if (P["grid"] != row_blocks * KS) fail("split plan", fmtv("grid %lld, row blocks %lld x %lld ranges", P["grid"], row_blocks, KS));
  if (P["lds_bytes"] != 2 * buf_bytes) fail("split plan", fmtv("lds %lld, buffers 2 x %lld", P["lds_bytes"], buf_bytes));
  if (GP % 4 || (KS > 1 && GK % 4)) fail("split plan", fmtv("pass %lld / range %lld groups not whole chunks", GP, GK));
  if (MP < M) fail("split plan", fmtv("token slots %lld < M %lld", MP, M));
  if (cdiv(G, GK) != KS) fail("split plan", fmtv("%lld ranges of %lld groups do not cover %lld groups", KS, GK, G));
  const int threads = 64 * NW;
  const int64_t kPartOffset = 8192 * 4;
  std::vector<int> arrivals(size_t(row_blocks), 0);
  for (int64_t b = 0; b < P["grid"]; ++b) {
    Buf lds("LDS", P["lds_bytes"], true);
    const int64_t ks = b % KS, rb = b / KS;
    const int64_t g0 = ks * GK;
    const int64_t ng = std::min<int64_t>(GK, G - g0);
    if (ng < 1) fail("split", fmtv("workgroup %lld: empty K range %lld", b, ks));
    const int64_t nchunks = cdiv(ng, 4), c0 = g0 / 4;
    if (g0 % 4) fail("split", "K range not on a chunk boundary");
    const int64_t npass = cdiv(ng, GP), cpp = GP / 4;
    if (!fp4) {  // zero cells of both buffers
      lds.write(GP * 16 * MP * 16, 16, "zero cell", -2);
      lds.write(buf_bytes + GP * 16 * MP * 16, 16, "zero cell", -2);
    }
    // Staging of pass ps: loads (load_raw), then the conversion into buffer ps & 1.
    auto stage = [&](int64_t ps) {
      const int64_t gb = g0 + ps * GP, npg = std::min<int64_t>(GP, ng - ps * GP);
      const int64_t base = (ps & 1) * buf_bytes;
      for (int item = 0; item < threads; ++item) {
        // Token slot fastest in the exact modes, lane quarter fastest with fp8 pieces.
        const int64_t m = fp4 ? (item >> 2) / GP : item % MP;
        const int q = fp4 ? (item & 3) : int((item / MP) & 3);
        const int64_t gl = fp4 ? (item >> 2) % GP : (item / MP) >> 2;
        const bool live = item < MP * GP * 4;
        const bool in = live && m < M && gl < npg;
        const int64_t src = in ? m * K + 128 * (gb + gl) + 8 * q : 0;
        for (int u = 0; u < 4; ++u) X.read(2 * (src + 32 * u), 16, "x (staging)");
        if (!live) continue;
        if (!fp4) {
          for (int u = 0; u < 4; ++u)
            lds.write(base + (((gl * 4 + u) * 4 + q) * MP + m) * 16, 16, "x cells", int32_t(ps));
        } else {
          const int64_t row = base + (gl * 2 * MP + (MP > 8 ? m : 2 * m)) * kRowBytes;
          const int64_t lrow = row + (MP > 8 ? MP : 1) * kRowBytes;
          const int qa = 2 * (q & 1), half = 16 * (q >> 1);
          lds.write(row + qa * 32 + half, 16, "x pieces", int32_t(ps));
          lds.write(row + (qa + 1) * 32 + half, 16, "x pieces", int32_t(ps));
          lds.write(lrow + qa * 32 + half, 16, "x pieces", int32_t(ps));
          lds.write(lrow + (qa + 1) * 32 + half, 16, "x pieces", int32_t(ps));
          lds.write(base + GP * 2 * MP * kRowBytes + (gl * MP + m) * 4 + q, 1, "x scales", int32_t(ps));
        }
      }
    };
    stage(0);
    // Sixteen tokens in passes of two chunks: the raw x of the pass after
    // the last is loaded too (zeros from clamped addresses, never converted).
    if (MP == 16 && GP == 8) {
      const int64_t gb = g0 + npass * GP, npg = std::min<int64_t>(GP, ng - npass * GP);
      for (int item = 0; item < threads; ++item) {
        // Token slot fastest in the exact modes, lane quarter fastest with fp8 pieces.
        const int64_t m = fp4 ? (item >> 2) / GP : item % MP;
        const int q = fp4 ? (item & 3) : int((item / MP) & 3);
        const int64_t gl = fp4 ? (item >> 2) % GP : (item / MP) >> 2;
        const bool in = item < MP * GP * 4 && m < M && gl < npg;
        const int64_t src = in ? m * K + 128 * (gb + gl) + 8 * q : 0;
        for (int u = 0; u < 4; ++u) X.read(2 * (src + 32 * u), 16, "x (staging past the range)");
      }
    }
    for (int64_t ps = 0; ps < npass; ++ps) {
      if (ps > 0) stage(ps);
      const int64_t base = (ps & 1) * buf_bytes;
      const int64_t png = std::min<int64_t>(GP, ng - ps * GP);
      for (int64_t cc = ps * cpp; cc < std::min<int64_t>(nchunks, (ps + 1) * cpp); ++cc) {
        const int64_t cl = cc - ps * cpp;
        const int64_t ngc = std::min<int64_t>(4, png - 4 * cl);
        for (int64_t gi = 0; gi < ngc; ++gi) {
          const int64_t gl = 4 * cl + gi;
          for (int lane = 0; lane < 64; ++lane) {
            const int qa = lane >> 4, r = lane & 15;
            if (fp4 && MP <= 8) {
              const int rr = r < 2 * MP ? r : 0;
              lds.read_tagged(base + (gl * 2 * MP + rr) * kRowBytes + qa * 32, 32, int32_t(ps), "x pieces read");
              lds.read_tagged(base + GP * 2 * MP * kRowBytes + (gl * MP + (rr >> 1)) * 4 + qa, 1, int32_t(ps),
                              "x scale read");
            } else if (fp4) {
              const int64_t xh = base + (gl * 2 * MP + r) * kRowBytes + qa * 32;
              lds.read_tagged(xh, 32, int32_t(ps), "x hi read");
              lds.read_tagged(xh + MP * kRowBytes, 32, int32_t(ps), "x lo read");
              lds.read_tagged(base + GP * 2 * MP * kRowBytes + (gl * MP + r) * 4 + qa, 1, int32_t(ps), "x scale read");
            } else {
              for (int uu = 0; uu < 4; ++uu) {
                if (r < MP)
                  lds.read_tagged(base + (((gl * 4 + uu) * 4 + qa) * MP + r) * 16, 16, int32_t(ps), "x cell read");
                else
                  lds.read_tagged(GP * 16 * MP * 16, 16, -2, "zero cell read");
              }
            }
          }
        }
      }
    }
    // Weights: the two-unit ring of every wave (chunk indices clamped to the range).
    for (int w = 0; w < NW; ++w) {
      const int64_t t0 = rb * NW * R + int64_t(w) * R;
      auto load = [&](int64_t c) {
        if (full) load_full(ms, fmt, R, t0, c0 + c);
        else load_unit(ms, fmt, R, t0, c0 + c, true);
      };
      load(0);
      load(std::min<int64_t>(1, nchunks - 1));
      for (int64_t c = 0; c < nchunks; c += 2)
        for (int h = 0; h < 2; ++h) load(std::min<int64_t>(c + h + 2, nchunks - 1));
      // This wave's outputs.
      for (int r = 0; r < R; ++r) {
        if (t0 + r >= ms.tiles) continue;
        for (int lane = 0; lane < 64; ++lane) {
          const int j = lane & 15, qa = lane >> 4;
          for (int e = 0; e < (fp4 && MP <= 8 ? 2 : 4); ++e) {
            const int64_t m = fp4 && MP <= 8 ? 2 * qa + e : 4 * qa + e;
            if (m >= M) continue;
            if (KS == 1) {
              int mi;
              int64_t t;
              ms.tile_ref(t0 + r, mi, t);
              ms.store_y(mi, t, j, m);
            } else {
              ws.write(kPartOffset + 4 * ((ks * M + m) * NV + 16 * (t0 + r) + j), 4, "partial sum store",
                       int32_t(1000 + ks));
            }
          }
        }
      }
    }
    if (KS == 1) continue;
    // Arrival: the last of the KS workgroups of the row block sums.
    ws.check(4 * rb, 4, "arrival counter");
    const uint32_t old = ws.u32(4 * rb);
    ws.set_u32(4 * rb, old + 1);
    if (old != uint32_t(KS - 1)) continue;
    const int64_t n0 = rb * NW * R * 16;
    const int64_t rows = std::min<int64_t>(NW * R * 16, NV - n0);
    const int64_t outs = M * rows;
    const int KR = KS <= 4 ? 4 : 8;
    for (int64_t base = 0; base < outs; base += 4 * threads)
      for (int th = 0; th < threads; ++th)
        for (int o = 0; o < 4; ++o) {
          const int64_t idx = std::min<int64_t>(base + o * threads + th, outs - 1);
          const int64_t pm = idx / rows, pn = n0 + idx % rows;
          for (int64_t k0 = 0; k0 < KS; k0 += KR)
            for (int k = 0; k < KR; ++k) {
              const int64_t kk = std::min<int64_t>(k0 + k, KS - 1);
              ws.read_tagged(kPartOffset + 4 * ((kk * M + pm) * NV + pn), 4, int32_t(1000 + kk), "partial sum load");
            }
          if (base + o * threads + th < outs) {
            int mi;
            int64_t t;
            ms.tile_ref(pn >> 4, mi, t);
            ms.store_y(mi, t, pn & 15, pm);
          }
        }
    ws.set_u32(4 * rb, 0);
  }
  for (int64_t rb = 0; rb < row_blocks && KS > 1; ++rb)
    if (ws.u32(4 * rb) != 0) fail("arrival counter", fmtv("row block %lld left at %lld", rb, ws.u32(4 * rb)));
}

// ------------------------------------------------------- k-slice kernel ----
// Wave w of a workgroup owns chunk w of K for the workgroup's T row tiles.
void kslice_kernel(Mats &ms, std::map<std::string, int64_t> &P, Buf &X) {
  const int fmt = ms.fmt;
  const int T = int(P["tiles_per_wave"]), NW = int(P["waves"]), D = int(P["ring"]);
  const bool fp4 = P["operands"] == 3;
  const int64_t M = ms.M, K = ms.K;
  if (P["whole_tiles"] != 1 || P["k_ranges"] != 1 || P["token_slots"] != 16)
    fail("kslice plan", "whole tiles, one K range and 16 token slots expected");
  if (K % 512 || NW != K / 512) fail("kslice plan", fmtv("%lld waves for K = %lld", NW, K));
  if (P["threads"] != 64 * NW) fail("kslice plan", fmtv("threads %lld", P["threads"]));
  if (P["grid"] != cdiv(ms.tiles, T)) fail("kslice plan", fmtv("grid %lld for %lld tiles of %lld", P["grid"], ms.tiles, T));
  if (P["lds_bytes"] != int64_t(T) * NW * 1024) fail("kslice plan", fmtv("lds %lld", P["lds_bytes"]));
  if (M < 1 || M > 16) fail("kslice plan", fmtv("M = %lld", M));
  for (int64_t b = 0; b < P["grid"]; ++b) {
    Buf lds("LDS", P["lds_bytes"], true);
    const int64_t t0 = b * T;
    for (int w = 0; w < NW; ++w) {
      // A operands: lane (qa, r) reads x of token r (row 0 past M).
      for (int lane = 0; lane < 64; ++lane) {
        const int qa = lane >> 4, r = lane & 15;
        const int64_t row = r < M ? r : 0;
        for (int g = 0; g < 4; ++g)
          for (int u = 0; u < 4; ++u) {
            const int64_t k = 512 * w + 128 * g + (fp4 ? 8 * qa + 32 * u : 32 * u + 8 * qa);
            X.read(2 * (row * K + k), 16, "x (A operand)");
          }
        if (fp4)  // the halves come from lanes of the same token
          for (int src : {16 * (qa >> 1) + r, 16 * (2 + (qa >> 1)) + r})
            if (src < 0 || src > 63) fail("kslice", "ds_bpermute source lane");
      }
      // Weights: a ring of D units, one per tile step, clamped to the last tile.
      for (int d = 0; d < D; ++d) load_full(ms, fmt, 1, std::min<int64_t>(t0 + std::min<int64_t>(d, T - 1), ms.tiles - 1), w);
      for (int t = 0; t + D < T; ++t) load_full(ms, fmt, 1, std::min<int64_t>(t0 + t + D, ms.tiles - 1), w);
      // This wave's sums into LDS.
      for (int t = 0; t < T; ++t)
        for (int lane = 0; lane < 64; ++lane) lds.write(16 * ((int64_t(t) * NW + w) * 64 + lane), 16, "wave sums", 7);
    }
    // After the barrier: each output (tile, lane, e) adds the NW waves' sums.
    for (int64_t o = 0; o < int64_t(T) * 256; ++o) {
      const int64_t t = o >> 8, ln = (o >> 2) & 63, e = o & 3;
      const int64_t m = 4 * (ln >> 4) + e;
      if (t0 + t >= ms.tiles || m >= M) continue;
      for (int w = 0; w < NW; ++w) lds.read_tagged(4 * (((t * NW + w) * 64 + ln) * 4 + e), 4, 7, "wave sum read");
      int mi;
      int64_t tt;
      ms.tile_ref(t0 + t, mi, tt);
      ms.store_y(mi, tt, ln & 15, m);
    }
  }
}

// -------------------------------------------------------- staged kernel ----
void staged_kernel(Mats &ms, std::map<std::string, int64_t> &P, Buf &X) {
  const int fmt = ms.fmt;
  const int MT = int(P["token_slots"]), R = int(P["tiles_per_wave"]), D = int(P["ring"]);
  // fp8 x fp4 operands: two pieces per token (bf16 x) or three (fp16 x, one token).
  const bool fp4 = P["operands"] == 3 || P["operands"] == 4, full = P["whole_tiles"] != 0;
  const int NPC = P["operands"] == 4 ? 3 : 2;
  const int S = int(P["waves_per_tile"]), Pw = 8 / S;
  const int64_t G = ms.G, M = ms.M, K = ms.K;
  const int64_t chunks = cdiv(G, 4);
  const int64_t SC = P["groups_per_pass"] / 4;
  const int64_t n_stages = cdiv(chunks, SC);
  const int64_t tilesets = cdiv(ms.tiles, R);
  const int64_t grid = P["grid"];
  const int64_t off_corr = P["lds0"], off_x = P["lds1"], off_red = P["lds2"];
  const int E = fp4 ? (MT == 1 ? NPC : 4) : (MT == 1 ? 1 : 4);
  const int kRowBytes = 144;
  if (NPC == 3 && MT != 1) fail("staged plan", "three pieces per token on more than one token slot");
  if (SC % S) fail("staged plan", "stage not a multiple of the K split");
  if (MT < M) fail("staged plan", fmtv("token slots %lld < M %lld", MT, M));
  const int64_t U = SC / S, KT = n_stages * U;
  const bool restage = n_stages > 1, lockstep = restage || S > 1;
  const int64_t rows_total = grid * Pw;
  // Every chunk of every tile set is multiplied exactly once.
  std::vector<int> cover(size_t(tilesets * chunks), 0);
  for (int64_t b = 0; b < grid; ++b) {
    Buf lds("LDS", P["lds_bytes"], true);
    if (!fp4 && MT < 16)
      for (int i = 0; i < 64 * MT; ++i) lds.write(16 * i, 16, "zero region", -2);
    // x staging of chunks [c0, c0 + nc) (all at once, or per stage).
    auto stage = [&](int64_t c0, int64_t nc, int32_t tag) {
      if (fp4) {
        const int64_t items = int64_t(MT) * 4 * nc * 4;
        for (int64_t it = 0; it < std::max<int64_t>(items, 512); ++it) {
          if (it >= items) break;
          const int q = int(it & 3);
          const int64_t rest = it >> 2, gl = rest % (4 * nc), m = rest / (4 * nc);
          const bool in = m < M && 4 * c0 + gl < G;
          const int64_t src = in ? m * K + 128 * (4 * c0 + gl) + 8 * q : 0;
          for (int u = 0; u < 4; ++u) X.read(2 * (src + 32 * u), 16, "x (staging)");
          const int64_t row = off_x + (gl * NPC * MT + NPC * m) * kRowBytes;
          const int qa = 2 * (q & 1), half = 16 * (q >> 1);
          for (int pc = 0; pc < NPC; ++pc) {
            lds.write(row + pc * kRowBytes + qa * 32 + half, 16, "x pieces", tag);
            lds.write(row + pc * kRowBytes + (qa + 1) * 32 + half, 16, "x pieces", tag);
          }
          lds.write(off_corr + (gl * MT + m) * 4 + q, 1, "x scales", tag);
        }
        // The first item of each thread was loaded before the weights
        // (threads past the items load item 0's address pattern too).
        for (int th = int(std::min<int64_t>(items, 512)); th < 512; ++th) {
          const int q = th & 3;
          const int64_t rest = th >> 2, gl = rest % (4 * nc), m = rest / (4 * nc);
          const bool in = m < M && 4 * c0 + gl < G;
          const int64_t src = in ? m * K + 128 * (4 * c0 + gl) + 8 * q : 0;
          for (int u = 0; u < 4; ++u) X.read(2 * (src + 32 * u), 16, "x (first item)");
        }
      } else {
        const int64_t cells = int64_t(MT) * nc * 64;
        for (int64_t base = 0; base < std::max<int64_t>(cells, 4 * 512); base += 512)
          for (int th = 0; th < 512; ++th) {
            const int64_t idx = base + th;
            const int64_t m = idx / (nc * 64), oct = idx - m * (nc * 64);
            const int64_t k = c0 * 512 + oct * 8;
            const bool in = idx < cells && k < K && m < M;
            X.read(2 * (in ? m * K + k : 0), 16, "x cell");
            if (idx < cells) {
              lds.write(off_x + (oct * MT + m) * 16, 16, "x cells", tag);
              if (fmt == 1 && (oct & 15) == 0) lds.write(off_corr + 4 * ((oct >> 4) * 16 + m), 4, "corrections", tag);
            }
          }
        if (fmt == 1)
          for (int64_t idx = 0; idx < nc * 4 * (16 - MT); ++idx) {
            const int64_t gs = idx / (16 - MT), m = MT + idx % (16 - MT);
            lds.write(off_corr + 4 * (gs * 16 + m), 4, "corrections", tag);
          }
      }
    };
    if (!restage) stage(0, chunks, 0);
    // Per wave: its position, sequence length and loads (loads touch no LDS).
    int64_t my_row[8], total[8];
    for (int w = 0; w < 8; ++w) {
      const int pr = w / S, s = w % S;
      my_row[w] = int64_t(pr) * grid + b;
      const int64_t iters = lockstep ? cdiv(tilesets, rows_total) : cdiv(tilesets - my_row[w], rows_total);
      total[w] = iters * KT;
      // The load cursor walks (it, st, kl) over total + D - 1 steps (every
      // step of the ring issues one load).
      const int64_t steps = cdiv(std::max<int64_t>(total[w], 0), D) * D + D - 1;
      for (int64_t i = 0; i < steps; ++i) {
        const int64_t it = i / KT, rem = i % KT, st = rem / U, kl = rem % U;
        const int64_t ch = st * SC + s + kl * S, t0 = (it * rows_total + my_row[w]) * R;
        const bool v = i < total[w] && it * rows_total + my_row[w] < tilesets && ch < chunks;
        if (full) load_full(ms, fmt, R, t0, v ? ch : 0);
        else load_unit(ms, fmt, R, t0, ch, v);
      }
    }
    // Compute steps in lockstep across the waves (restaging and the K-split
    // sums are workgroup barriers in the kernel).
    int64_t max_total = 0;
    for (int w = 0; w < 8; ++w) max_total = std::max(max_total, total[w]);
    for (int64_t i = 0; i < max_total; ++i) {
      const int64_t it = i / KT, rem = i % KT, st = rem / U, kl = rem % U;
      const int32_t tag = restage ? int32_t(st) : 0;
      if (restage && kl == 0) stage(st * SC, std::min<int64_t>(SC, chunks - st * SC), int32_t(st));
      for (int w = 0; w < 8; ++w) {
        if (i >= total[w]) continue;
        const int s = w % S;
        const int64_t t0 = (it * rows_total + my_row[w]) * R;
        const int64_t ch = st * SC + s + kl * S;
        const bool v = it * rows_total + my_row[w] < tilesets && ch < chunks;
        if (v) {
          ++cover[size_t((it * rows_total + my_row[w]) * chunks + ch)];
          const int64_t c_local = s + kl * S;
          for (int lane = 0; lane < 64; ++lane) {
            const int j = lane & 15, q = lane >> 4;
            if (fp4) {
              const int rr = j < NPC * MT ? j : 0;
              for (int g = 0; g < 4; ++g) {
                if (4 * ch + g >= G) break;
                const int64_t xa = off_x + (c_local * 4 * NPC * MT + rr) * kRowBytes + q * 32 + g * NPC * MT * kRowBytes;
                lds.read_tagged(xa, 32, tag, "x pieces read");
                lds.read_tagged(off_corr + (c_local * 4 * MT + rr / NPC) * 4 + q + g * MT * 4, 1, tag,
                                "x scale read");
              }
            } else {
              const bool xact = j < MT;
              for (int g = 0; g < 4; ++g) {
                if (fmt == 1) lds.read_tagged(off_corr + 4 * (c_local * 64 + 4 * q + g * 16), 4 * (E == 1 ? 1 : 4),
                                              tag, "correction read");
                for (int uu = 0; uu < 4; ++uu) {
                  if (xact)
                    lds.read_tagged(off_x + (c_local * 64 * MT + q * MT + j) * 16 + (g * 16 + 4 * uu) * MT * 16, 16,
                                    tag, "x cell read");
                  else
                    lds.read_tagged((g * 16 + 4 * uu) * MT * 16, 16, -2, "zero region read");
                }
              }
            }
          }
        }
        const bool k_last = st == n_stages - 1 && kl == U - 1;
        if (!k_last) continue;
        const bool ts_ok = t0 < ms.tiles;
        if (S > 1)
          for (int r = 0; r < R; ++r)
            for (int e = 0; e < E; ++e)
              for (int lane = 0; lane < 64; ++lane)
                lds.write(off_red + 4 * (((int64_t(w) * R + r) * E + e) * 64 + lane), 4, "reduction", -3);
        if ((S == 1 || s == 0) && ts_ok)
          for (int r = 0; r < R; ++r) {
            if (t0 + r >= ms.tiles) continue;
            int mi;
            int64_t t;
            ms.tile_ref(t0 + r, mi, t);
            for (int lane = 0; lane < 64; ++lane) {
              const int j = lane & 15, q = lane >> 4;
              if (fp4 && NPC == 3) {  // three pieces of token 0 in lane quarter 0
                if (q == 0) ms.store_y(mi, t, j, 0);
                continue;
              }
              for (int e = 0; e < (fp4 ? E / 2 : E); ++e) {
                const int64_t m = fp4 ? 2 * q + e : 4 * q + e;
                if (m < M) ms.store_y(mi, t, j, m);
              }
            }
          }
      }
    }
  }
  for (int64_t ts = 0; ts < tilesets; ++ts)
    for (int64_t c = 0; c < chunks; ++c)
      if (cover[size_t(ts * chunks + c)] != 1)
        fail("staged", fmtv("tile set %lld chunk %lld multiplied %lld times", ts, c, cover[size_t(ts * chunks + c)]));
}

// ---------------------------------------------------------- wide kernel ----
void wide_kernel(Mats &ms, std::map<std::string, int64_t> &P, Buf &X) {
  const int fmt = ms.fmt;
  const int R = int(P["tiles_per_wave"]), D = int(P["ring"]), S = int(P["waves_per_tile"]), Pw = 8 / S;
  const int64_t GS = P["groups_per_range"], grid = P["grid"];
  const int64_t G = ms.G, M = ms.M, K = ms.K;
  const int64_t tilesets = cdiv(ms.tiles, R), rows_total = grid * Pw;
  const int64_t unit = fmt == 1 ? 16 : 32;
  for (int64_t b = 0; b < grid; ++b)
    for (int w = 0; w < 8; ++w) {
      const int pr = w / S, s = w % S;
      const int64_t my_row = int64_t(pr) * grid + b;
      const int64_t iters = cdiv(tilesets, rows_total), total = iters * GS, g_begin = s * GS;
      auto tile0 = [&](int64_t i) { return ((i / GS) * rows_total + my_row) * R; };
      auto valid = [&](int64_t i) { return (i / GS) * rows_total + my_row < tilesets && g_begin + i % GS < G; };
      const int64_t steps = cdiv(total, D) * D + D - 1;
      for (int64_t i = 0; i < steps; ++i) {
        const bool v = i < total && valid(i);
        const int64_t g = v ? g_begin + i % GS : 0;
        const int64_t c = g >> 2, gc = g & 3, Gc = std::min<int64_t>(4, G - 4 * c);
        for (int lane = 0; lane < 64; ++lane) {
          const int j = lane & 15, q = lane >> 4;
          const int64_t xr = (j < M ? j * K : 0) + 128 * g + 8 * q;
          for (int st = 0; st < 4; ++st) X.read(2 * (xr + 32 * st), 16, "x (registers)");
          for (int r = 0; r < R; ++r) {
            int mi;
            int64_t t;
            ms.tile_ref(std::min<int64_t>(tile0(i) + r, ms.tiles - 1), mi, t);
            const int64_t RT = ms.rows_of(mi, t), jj = std::min<int64_t>(j, RT - 1);
            const int64_t blk = 16 * t * G * unit + RT * 4 * c * unit;
            if (fmt == 1) ms.W[mi]->read(blk + 4 * ((q * RT + jj) * Gc + gc), 4, "weights");
            else {
              const int64_t hh = gc >> 1, Gh = std::min<int64_t>(2, Gc - 2 * hh);
              ms.W[mi]->read(blk + 4 * (RT * 16 * hh + ((q * RT + jj) * Gh + (gc - 2 * hh)) * 2), 8, "weights");
            }
            ms.W[mi]->read(ms.sc_off(mi) + 2 * (16 * t * G + RT * 4 * c + jj * Gc + gc), 2, "scales");
          }
        }
      }
      for (int64_t i = 0; i < total; ++i) {
        if (i % GS != GS - 1) continue;
        const int64_t t0 = tile0(i);
        const bool ts_ok = (i / GS) * rows_total + my_row < tilesets;
        if (!ts_ok || (S > 1 && s != 0)) continue;
        for (int r = 0; r < R; ++r) {
          if (t0 + r >= ms.tiles) continue;
          int mi;
          int64_t t;
          ms.tile_ref(t0 + r, mi, t);
          for (int lane = 0; lane < 64; ++lane)
            for (int e = 0; e < 4; ++e) {
              const int64_t m = 4 * (lane >> 4) + e;
              if (m < M) ms.store_y(mi, t, lane & 15, m);
            }
        }
      }
    }
}

// ----------------------------------------------------------- tq5 kernels ----
struct T5 {
  int64_t s_full, L_tail, b_tail, rowbytes, nseg;
  explicit T5(int64_t K) {
    s_full = K / 640;
    L_tail = K - 640 * s_full;
    b_tail = (L_tail + 4) / 5;
    rowbytes = 128 * s_full + b_tail;
    nseg = s_full + (L_tail > 0 ? 1 : 0);
  }
};

// Tail operand bytes of group i, k-step u (t5_tail_operand) of tile vt.
void t5_tail(Mats &ms, const T5 &g5, int64_t vt, int64_t i, int u) {
  int mi;
  int64_t t;
  ms.tile_ref(vt, mi, t);
  const int64_t RT = ms.rows_of(mi, t);
  for (int lane = 0; lane < 64; ++lane) {
    const int j = lane & 15, q = lane >> 4;
    const int64_t jj = std::min<int64_t>(j, RT - 1);
    const int64_t rb = 16 * t * g5.rowbytes + RT * 128 * g5.s_full + jj * g5.b_tail;
    for (int e = 0; e < 8; ++e) {
      const int64_t kt = 128 * i + 32 * u + 8 * q + e;
      if (kt >= g5.L_tail) fail("tq5 tail", fmtv("trit %lld of a %lld-trit tail", kt, g5.L_tail));
      ms.W[mi]->read(rb + kt % g5.b_tail, 1, "tq5 tail byte");
    }
  }
}

void tq5_x_regs(Mats &ms, Buf &X, int64_t g, bool valid) {
  for (int lane = 0; lane < 64; ++lane) {
    const int j = lane & 15, q = lane >> 4;
    const bool tok = valid && j < ms.M;
    const int64_t xr = (tok ? j * ms.K + 128 * g : 0) + 8 * q;
    for (int u = 0; u < 4; ++u) X.read(2 * (xr + 32 * u), 16, "x (registers)");
  }
}

void tq5_kernel(Mats &ms, std::map<std::string, int64_t> &P, Buf &X) {
  const T5 g5(ms.K);
  const int R = int(P["tiles_per_wave"]), S = int(P["waves_per_tile"]), Pw = 8 / S;
  const int64_t SS = P["groups_per_range"] / 5, grid = P["grid"], G = ms.G, M = ms.M;
  const int64_t tilesets = cdiv(ms.tiles, R), rows_total = grid * Pw;
  for (int64_t b = 0; b < grid; ++b)
    for (int w = 0; w < 8; ++w) {
      const int pr = w / S, s = w % S;
      const int64_t my_row = int64_t(pr) * grid + b;
      const int64_t iters = cdiv(tilesets, rows_total), total = iters * SS, seg0 = s * SS;
      auto tile0 = [&](int64_t i) { return ((i / SS) * rows_total + my_row) * R; };
      auto segment = [&](int64_t i) { return seg0 + i % SS; };
      auto valid = [&](int64_t i) {
        return i < total && (i / SS) * rows_total + my_row < tilesets && segment(i) < g5.nseg;
      };
      auto load = [&](int64_t i) {  // t5_load
        if (!valid(i)) return;
        const int64_t seg = segment(i);
        for (int r = 0; r < R; ++r) {
          const int64_t vt = tile0(i) + r;
          if (vt >= ms.tiles) continue;
          int mi;
          int64_t t;
          ms.tile_ref(vt, mi, t);
          const int64_t RT = ms.rows_of(mi, t);
          const int64_t Gs = std::min<int64_t>(5, G - 5 * seg);
          for (int lane = 0; lane < 64; ++lane) {
            const int j = lane & 15, q = lane >> 4;
            const int64_t jj = std::min<int64_t>(j, RT - 1);
            if (seg < g5.s_full) {
              const int64_t sb = 16 * t * g5.rowbytes + RT * 128 * seg + (q * RT + jj) * 16;
              ms.W[mi]->read(sb, 16, "tq5 segment bytes");
              ms.W[mi]->read(sb + RT * 64, 16, "tq5 segment bytes");
            }
            for (int k = 0; k < 5; ++k)
              ms.W[mi]->read(ms.sc_off(mi) + 2 * (16 * t * G + RT * 5 * seg + jj * Gs + std::min<int64_t>(k, Gs - 1)),
                             2, "tq5 scales");
          }
        }
      };
      load(0);
      tq5_x_regs(ms, X, 5 * segment(0), valid(0));
      for (int64_t i = 0; i < total; ++i) {
        load(i + 1);
        if (valid(i)) {
          const int64_t seg = segment(i), ng = std::min<int64_t>(5, G - 5 * seg);
          const int64_t gnext = 5 * segment(i + 1);
          if (seg < g5.s_full) {
            for (int gi = 0; gi < 5; ++gi) {
              if (gi < 4) tq5_x_regs(ms, X, 5 * seg + gi + 1, true);
              else tq5_x_regs(ms, X, gnext, valid(i + 1));
            }
          } else {
            for (int64_t gi = 0; gi < ng; ++gi) {
              tq5_x_regs(ms, X, gi + 1 < ng ? 5 * seg + gi + 1 : gnext, gi + 1 < ng ? true : valid(i + 1));
              for (int u = 0; u < 4; ++u)
                for (int r = 0; r < R; ++r) {
                  const int64_t vt = tile0(i) + r < ms.tiles ? tile0(i) + r : 0;
                  t5_tail(ms, g5, vt, gi, u);
                }
            }
          }
        } else {
          tq5_x_regs(ms, X, 5 * segment(i + 1), valid(i + 1));
        }
        if (i % SS == SS - 1) {
          const bool ts_ok = (i / SS) * rows_total + my_row < tilesets;
          if (!ts_ok || (S > 1 && s != 0)) continue;
          const int64_t t0 = tile0(i);
          for (int r = 0; r < R; ++r) {
            if (t0 + r >= ms.tiles) continue;
            int mi;
            int64_t t;
            ms.tile_ref(t0 + r, mi, t);
            for (int lane = 0; lane < 64; ++lane)
              for (int e = 0; e < 4; ++e) {
                const int64_t m = 4 * (lane >> 4) + e;
                if (m < M) ms.store_y(mi, t, lane & 15, m);
              }
          }
        }
      }
    }
}

void tq5_one_kernel(Mats &ms, std::map<std::string, int64_t> &P, Buf &X) {
  const T5 g5(ms.K);
  const int R = int(P["tiles_per_wave"]), S = int(P["waves_per_tile"]), Pw = 8 / S, D = 3;
  const int64_t SS = P["groups_per_range"] / 5, grid = P["grid"], G = ms.G, K = ms.K;
  const int64_t tilesets = cdiv(ms.tiles, R), rows_total = grid * Pw;
  if (ms.M != 1) fail("tq5 one-token plan", fmtv("M = %lld", ms.M));
  if (P["lds_bytes"] != K * 2 + 16) fail("tq5 one-token plan", "LDS is not x plus one zero cell");
  for (int64_t b = 0; b < grid; ++b) {
    Buf lds("LDS", P["lds_bytes"], true);
    const int64_t cells = K / 8;
    for (int th = 0; th < 512; ++th)
      for (int c = 0; c < 4; ++c) X.read(16 * std::min<int64_t>(th + c * 512, cells - 1), 16, "x (first cells)");
    for (int64_t cell = 0; cell < cells; ++cell) {
      if (cell >= 4 * 512) X.read(16 * cell, 16, "x cells");
      lds.write(16 * cell, 16, "x", 0);
    }
    lds.write(K * 2, 16, "zero cell", -2);
    for (int w = 0; w < 8; ++w) {
      const int pr = w / S, s = w % S;
      const int64_t my_row = int64_t(pr) * grid + b;
      const int64_t iters = cdiv(tilesets, rows_total), total = iters * SS, seg0 = s * SS;
      auto tile0 = [&](int64_t i) { return ((i / SS) * rows_total + my_row) * R; };
      auto segment = [&](int64_t i) { return seg0 + i % SS; };
      auto valid = [&](int64_t i) {
        return i < total && (i / SS) * rows_total + my_row < tilesets && segment(i) < g5.nseg;
      };
      const int64_t steps = cdiv(total, D) * D + D - 1;
      for (int64_t i = 0; i < steps; ++i) {  // t5_resolve + t5_load_ts
        const int64_t seg = valid(i) ? segment(i) : seg0;
        const int64_t sf = std::max<int64_t>(std::min<int64_t>(seg, g5.s_full - 1), 0);
        const int64_t ss = std::max<int64_t>(std::min<int64_t>(seg, g5.nseg - 1), 0);
        const int64_t Gs = std::min<int64_t>(5, G - 5 * ss);
        for (int r = 0; r < R; ++r) {
          int mi;
          int64_t t;
          ms.tile_ref(std::min<int64_t>(tile0(i) + r, ms.tiles - 1), mi, t);
          const int64_t RT = ms.rows_of(mi, t);
          for (int lane = 0; lane < 64; ++lane) {
            const int j = lane & 15, q = lane >> 4;
            const int64_t jj = std::min<int64_t>(j, RT - 1);
            const int64_t tw = 16 * t * g5.rowbytes;
            const int64_t sb = g5.s_full > 0 ? tw + RT * 128 * sf + (q * RT + jj) * 16 : tw;
            const int64_t hb = g5.s_full > 0 ? RT * 64 : 0;
            ms.W[mi]->read(sb, 16, "tq5 segment bytes");
            ms.W[mi]->read(sb + hb, 16, "tq5 segment bytes");
            for (int k = 0; k < 5; ++k)
              ms.W[mi]->read(ms.sc_off(mi) + 2 * (16 * t * G + RT * 5 * ss + jj * Gs + std::min<int64_t>(k, Gs - 1)), 2,
                             "tq5 scales");
          }
        }
      }
      for (int64_t i = 0; i < total; ++i) {
        if (valid(i)) {
          const int64_t seg = segment(i), ng = std::min<int64_t>(5, G - 5 * seg);
          for (int64_t gi = 0; gi < (seg < g5.s_full ? 5 : ng); ++gi) {
            for (int lane = 0; lane < 64; ++lane) {  // t5_lds_x
              const int j = lane & 15, q = lane >> 4;
              const int64_t base = j == 0 ? (128 * (5 * seg + gi) + 8 * q) * 2 : K * 2;
              for (int u = 0; u < 4; ++u)
                lds.read_tagged(base + (j == 0 ? 64 : 0) * u, 16, j == 0 ? 0 : -2, "x read");
            }
            if (seg >= g5.s_full)
              for (int u = 0; u < 4; ++u)
                for (int r = 0; r < R; ++r) t5_tail(ms, g5, tile0(i) + r < ms.tiles ? tile0(i) + r : 0, gi, u);
          }
        }
        if (i % SS == SS - 1) {
          const bool ts_ok = (i / SS) * rows_total + my_row < tilesets;
          if (!ts_ok || (S > 1 && s != 0)) continue;
          const int64_t t0 = tile0(i);
          for (int r = 0; r < R; ++r) {
            if (t0 + r >= ms.tiles) continue;
            int mi;
            int64_t t;
            ms.tile_ref(t0 + r, mi, t);
            for (int lane = 0; lane < 64; ++lane)
              if (4 * (lane >> 4) == 0) ms.store_y(mi, t, lane & 15, 0);
          }
        }
      }
    }
  }
}

// --------------------------------------------------------------- GEMM ----
void gemm_kernel(Mats &ms, std::map<std::string, int64_t> &P, Buf &X, Buf &ws) {
  const int fmt = ms.fmt;
  const int64_t M = ms.M, N = ms.N[0], K = ms.K, G = ms.G;
  const int NB = fmt == 3 ? 2 : 4, NWN = 4, BN = 16 * NB * NWN, kBM = 128;
  const int XB = 32 / (2 * NWN), H = NB / 2;
  const bool XP = P["x_pieces"] != 0;
  const int64_t tiles_m = cdiv(M, kBM), tiles_n = cdiv(N, BN), tiles = tiles_m * tiles_n;
  const int64_t items = tiles * G, per = P["items_per_wg"], grid = P["grid"];
  const int64_t kCounterBytes = 64 << 10;
  const int64_t piece_floats = 2 * NWN * 64 * 16 * NB;
  const T5 g5(K);
  const int64_t last_chunk_groups = G - 4 * ((G - 1) / 4);
  Buf &W = *ms.W[0];
  const int64_t sc0 = ms.sc_off(0);
  // fp8 x pieces: converted by the pre-pass into the workspace.
  int64_t xp_off = 0, xs_off = 0;
  if (XP) {
    const int64_t slots = P["slots"];
    xp_off = (kCounterBytes + slots * 2 * piece_floats * 4 + 255) / 256 * 256;
    xs_off = xp_off + tiles_m * G * 32768;
    const int64_t xitems = tiles_m * kBM * G * 4;
    if (xs_off + tiles_m * G * 512 > ws.n) fail("gemm x pieces", "workspace too small");
    for (int64_t item = 0; item < xitems; ++item) {  // x_pieces_kernel
      const int r = int(item & 15), q = int((item >> 4) & 3);
      const int64_t rest = item >> 6, mb = rest & 7, blk = rest >> 3;
      const int64_t g = blk % G, mt = blk / G, m = mt * 128 + mb * 16 + r;
      const bool in = m < M;
      const int64_t src = in ? m * K + 128 * g + 8 * q : 0;
      for (int u = 0; u < 4; ++u) X.read(2 * (src + 32 * u), 16, "x (pieces pre-pass)");
      const int64_t bb = xp_off + blk * 32768 + mb * 4096 + (q >> 1) * 1024;
      const int l0 = 16 * (2 * (q & 1)) + r, l1 = l0 + 16;
      ws.write(bb + l0 * 16, 16, "x pieces", 7);
      ws.write(bb + l1 * 16, 16, "x pieces", 7);
      ws.write(bb + 2048 + l0 * 16, 16, "x pieces", 7);
      ws.write(bb + 2048 + l1 * 16, 16, "x pieces", 7);
      ws.write(xs_off + (blk * 8 + mb) * 64 + 16 * q + r, 1, "x piece scales", 7);
    }
  }
  if (per < 1 || grid * per < items) fail("gemm plan", fmtv("%lld x %lld items do not cover %lld", grid, per, items));
  if (per != G) {
    if (grid != cdiv(items, per)) fail("gemm plan", fmtv("grid %lld for %lld items of %lld", grid, items, per));
    if (kCounterBytes + grid * 2 * piece_floats * 4 > ws.n) fail("gemm plan", "workspace holds no pieces");
  } else if (grid != tiles) {
    fail("gemm plan", fmtv("whole tiles: grid %lld, tiles %lld", grid, tiles));
  }
  auto col_block = [&](int64_t nt, int wn, int nb, int64_t &T, int64_t &RR) {
    const int64_t n = nt * BN + int64_t(wn) * 16 * NB + 16 * nb;
    const int64_t R = n < N ? std::min<int64_t>(16, N - n) : 0;
    T = R > 0 ? n / 16 : 0;
    RR = R > 0 ? R : 1;
  };
  // The loads of item (tile, g) (feed_issue), for every wave and lane.
  auto issue = [&](int64_t tile, int64_t g, bool raw) {
    const int64_t mt = tile % tiles_m, nt = tile / tiles_m;
    for (int wave = 0; wave < 8; ++wave) {
      const int wm = wave / NWN, wn = wave % NWN;
      for (int lane = 0; lane < 64; ++lane) {
        const int j = lane & 15, q = lane >> 4;
        if (fmt != 3) {
          const int64_t c = g >> 2, gc = g & 3;
          const int64_t Gc = 4 * c + 4 > G ? last_chunk_groups : 4;
          const int64_t hh = gc >> 1, Gh = std::min<int64_t>(2, Gc - 2 * hh);
          for (int i = 0; i < H; ++i) {
            int64_t T, RR;
            col_block(nt, wn, H * wm + i, T, RR);
            const int64_t woff = q * RR + std::min<int64_t>(j, RR - 1);
            if (fmt == 1) W.read(16 * T * G * 16 + RR * 64 * c + 4 * gc + 4 * woff * Gc, 4, "gemm weights");
            else {
              const int64_t a = 16 * T * G * 32 + RR * (128 * c + 64 * hh) + 8 * (gc - 2 * hh) + 8 * woff * Gh;
              W.read(a, 4, "gemm weights");
              W.read(a + 4, 4, "gemm weights");
            }
          }
        }
        const int Wc = fmt == 3 ? 5 : 4;
        const int64_t sc = g / Wc, gs = g - Wc * sc, Gs = std::min<int64_t>(Wc, G - Wc * sc);
        int64_t T, RR;
        col_block(nt, wn, H * wm + ((lane >> 4) % H), T, RR);
        const int64_t sjj = std::min<int64_t>(j, RR - 1);
        W.read(sc0 + 32 * T * G + 2 * (RR * Wc * sc + sjj * Gs + gs), 2, "gemm scales");
        if (fmt == 3) {
          const int64_t seg = g / 5;
          if (raw && seg < g5.s_full)
            for (int i = 0; i < H; ++i) {
              int64_t T2, RR2;
              col_block(nt, wn, H * wm + i, T2, RR2);
              const int64_t woff = q * RR2 + std::min<int64_t>(j, RR2 - 1);
              const int64_t sb = 16 * T2 * g5.rowbytes + woff * 16 + RR2 * 128 * seg;
              for (int h = 0; h < 2; ++h) W.read(sb + h * RR2 * 64, 16, "gemm tq5 segment bytes");
            }
        }
        if (XP) {
          const int64_t item = mt * G + g;
          if (wave < 2) ws.read_tagged(xs_off + item * 512 + wave * 256 + lane * 4, 4, 7, "gemm x piece scales");
          for (int i = 0; i < XB; ++i)
            ws.read_tagged(xp_off + item * 32768 + lane * 16 + (wave * XB + i) * 1024, 16, 7, "gemm x pieces");
        } else {
          for (int i = 0; i < XB; ++i) {
            const int64_t row = std::min<int64_t>(mt * kBM + 16 * (wave * (XB / 4) + (i >> 2)) + j, M - 1);
            X.read(2 * (row * K + 8 * q + 128 * g + 32 * (i & 3)), 16, "gemm x");
          }
        }
      }
    }
  };
  auto tail = [&](int64_t nt, int64_t g) {  // tail-segment operand bytes
    for (int wave = 0; wave < 8; ++wave)
      for (int nb = 0; nb < NB; ++nb) {
        const int wn = wave % NWN;
        const int64_t n = nt * BN + int64_t(wn) * 16 * NB + 16 * nb;
        const int64_t R = n < N ? std::min<int64_t>(16, N - n) : 0;
        for (int lane = 0; lane < 64; ++lane) {
          const int j = lane & 15, q = lane >> 4;
          const int64_t jj = std::min<int64_t>(j, std::max<int64_t>(R - 1, 0));
          const int64_t T = R > 0 ? n / 16 : 0, RR = R > 0 ? R : 1;
          const int64_t tb = 16 * T * g5.rowbytes + RR * 128 * g5.s_full + jj * g5.b_tail;
          for (int u = 0; u < 4; ++u)
            for (int e = 0; e < 8; ++e) {
              const int64_t kt = 128 * (g - 5 * g5.s_full) + 32 * u + 8 * q + e;
              W.read(tb + kt % g5.b_tail, 1, "gemm tq5 tail byte");
            }
        }
      }
  };
  auto store_tile = [&](int64_t mt, int64_t nt) {
    for (int wave = 0; wave < 8; ++wave) {
      const int wm = wave / NWN, wn = wave % NWN;
      for (int lane = 0; lane < 64; ++lane) {
        const int j = lane & 15, q = lane >> 4;
        for (int mb = 0; mb < 4; ++mb)
          for (int nb = 0; nb < NB; ++nb) {
            const int64_t n = nt * BN + int64_t(wn) * 16 * NB + 16 * nb + j;
            if (n >= N) continue;
            for (int e = 0; e < 4; ++e) {
              const int64_t m = mt * kBM + wm * 64 + 16 * mb + 4 * q + e;
              if (m < M) ms.store_y(0, n / 16, n % 16, m);
            }
          }
      }
    }
  };
  std::vector<int> arrivals(size_t(tiles), 0);
  for (int64_t b = 0; b < grid; ++b) {
    int64_t n, first_tile, g0, wf0, wl0, wf1, wl1;
    if (per == G) {
      n = G; first_tile = b; g0 = 0; wf0 = wl0 = wf1 = wl1 = b;
    } else {
      const int64_t i0 = b * per, i1 = std::min(i0 + per, items);
      if (i0 >= i1) continue;
      n = i1 - i0;
      first_tile = i0 / G;
      const int64_t last_tile = (i1 - 1) / G;
      g0 = i0 - first_tile * G;
      wf0 = first_tile * G / per;
      wl0 = (first_tile * G + G - 1) / per;
      wf1 = last_tile * G / per;
      wl1 = (last_tile * G + G - 1) / per;
    }
    // Items in order; the feed runs two ahead and repeats the last item.
    int64_t ft = first_tile, fg = g0;
    int64_t fit = 0;
    auto raw_for = [&]() { return fmt == 3 && (fit == 0 || fg % 5 == 0); };
    auto advance_feed = [&]() {
      if (fit + 1 < n) {
        if (++fg == G) { fg = 0; ++ft; }
        ++fit;
      }
    };
    issue(ft, fg, raw_for());
    advance_feed();
    issue(ft, fg, raw_for());
    advance_feed();
    int64_t tile = first_tile, g = g0, g_begin = g0;
    for (int64_t it = 0; it < n; ++it) {
      issue(ft, fg, raw_for());
      advance_feed();
      const bool first = it == 0 || g == 0, last = it == n - 1 || g == G - 1;
      if (first) g_begin = g;
      if (fmt == 3 && g / 5 >= g5.s_full) tail(tile / tiles_m, g);
      if (last) {
        const int64_t mt = tile % tiles_m, nt = tile / tiles_m;
        if (g_begin == 0 && g == G - 1) {
          store_tile(mt, nt);
        } else {
          const int which = tile == first_tile ? 0 : 1;
          const int64_t wf = which ? wf1 : wf0, wl = which ? wl1 : wl0;
          const int64_t piece = kCounterBytes + 4 * ((b * 2 + which) * piece_floats);
          for (int64_t f = 0; f < piece_floats; ++f) ws.write(piece + 4 * f, 4, "gemm piece store", int32_t(b * 2 + which));
          if (tile >= kCounterBytes / 4) fail("gemm counters", fmtv("tile %lld", tile));
          const uint32_t old = ws.u32(4 * tile);
          ws.set_u32(4 * tile, old + 1);
          if (old == uint32_t(wl - wf)) {
            for (int64_t w2 = wf; w2 <= wl; ++w2) {
              const int wh = (w2 * per / G) == tile ? 0 : 1;
              const int64_t pc = kCounterBytes + 4 * ((w2 * 2 + wh) * piece_floats);
              for (int64_t f = 0; f < piece_floats; ++f)
                ws.read_tagged(pc + 4 * f, 4, int32_t(w2 * 2 + wh), "gemm piece load");
            }
            store_tile(mt, nt);
            ws.set_u32(4 * tile, 0);
          }
        }
      }
      if (++g == G) { g = 0; ++tile; }
    }
  }
  for (int64_t t = 0; t < tiles && per != G; ++t)
    if (ws.u32(4 * t) != 0) fail("gemm counter", fmtv("tile %lld left at %lld", t, ws.u32(4 * t)));
}

}  // namespace

int main(int argc, char **argv) {
  std::map<std::string, int64_t> P;
  std::string kernel;
  std::vector<int64_t> Ns;
  for (int i = 1; i < argc; ++i) {
    const std::string a = argv[i];
    const size_t eq = a.find('=');
    if (eq == std::string::npos) fail("args", a);
    const std::string k = a.substr(0, eq), v = a.substr(eq + 1);
    if (k == "kernel") kernel = v;
    else if (k == "N") Ns.push_back(std::atoll(v.c_str()));
    else P[k] = std::atoll(v.c_str());
  }
  Mats ms;
  ms.fmt = int(P["fmt"]);
  ms.nmat = 0;
  for (int64_t n : Ns)
    if (n > 0) ms.N[ms.nmat++] = n;
  ms.K = P["K"];
  ms.M = P["M"];
  ms.ysz = P["y_f16"] ? 2 : 4;
  ms.init();
  Buf X("X", ms.M * ms.K * 2);
  Buf ws("workspace", P["ws_bytes"], true);
  if (kernel == "gemv_split") split_kernel(ms, P, X, ws);
  else if (kernel == "gemv_staged") staged_kernel(ms, P, X);
  else if (kernel == "gemv_wide") wide_kernel(ms, P, X);
  else if (kernel == "gemv_kslice") kslice_kernel(ms, P, X);
  else if (kernel == "gemv_tq5") tq5_kernel(ms, P, X);
  else if (kernel == "gemv_tq5_one") tq5_one_kernel(ms, P, X);
  else if (kernel == "gemm") gemm_kernel(ms, P, X, ws);
  else fail("args", "unknown kernel " + kernel);
  ms.check_outputs();
  std::printf("ok\n");
  return 0;
}
