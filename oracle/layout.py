"""Packed weight formats and the device layout, written out element by element (oracle).

TEST INFRASTRUCTURE ONLY: nothing in the product imports this package.

What the pages fix
------------------
* Binary g128: one sign bit per weight, bit 0 -> -scale and bit 1 -> +scale,
  one FP16 scale per 128 weights, 1 + 16/128 = 1.125 bits/weight
  (lnrk.cn page, "Binary g128 weight representation" section; aberweb.com
  page, section 4.1 and Table 2).
* Ternary g128: weights in {-1, 0, +1}, one FP16 scale per 128 weights
  (ksqn.cn page, first technical section), shipped in 2-bit slots (same page,
  "current limitations"); the dense alternative packs 5 trits per byte,
  3^5 = 243 <= 256 (cnblogs.com page, section 2.4).

Readings taken where the pages are silent (each is listed in the design notes):
* a group is 128 consecutive weights along K inside one row;
* a 2-bit slot holds the code c = t + 1 (0 -> -1, 1 -> 0, 2 -> +1; 3 is
  invalid); a base-3 byte holds digits d_i = t_i + 1 little-endian
  (value = sum d_i 3^i, so a valid byte is 0..242);
* the blob is headerless: plane A (signs / codes / trit bytes) followed by
  plane B (the N*K/128 FP16 scales); no padding.

Device layout v2 (the arrangement the GPU kernels read)
-------------------------------------------------------
Plane A:
Rows are cut into tiles of 16 (tile T holds rows 16T .. 16T+R_T-1,
R_T = min(16, N-16T)); tiles are stored one after another.  Inside a tile the
groups are cut into chunks of 4 (chunk c holds groups 4c .. 4c+G_c-1,
G_c = min(4, G-4c)).  A weight at column k of its group is addressed by
u = k//32, q = (k//8) % 4, e = k % 8 (k here is the offset inside the group).

q1: unit (row, group) = 16 bytes.  Chunk c of tile T starts at byte
    T*16*G*16 + R_T*4c*16 and is a list of 32-bit little-endian words indexed
    ((q*R_T + j)*G_c + g); word (q, j, g) holds the 32 bits of row 16T+j,
    group 4c+g with that q, at bit position
        16*(e%2) + 15 - ((e//2)%2) - 2*(2u + (e//2)//2).
tq2: unit = 32 bytes.  Chunk c of tile T starts at T*16*G*32 + R_T*4c*32 and
    holds two half-blocks hh = 0, 1 (groups {2hh, 2hh+1} of the chunk,
    G_h = min(2, G_c-2hh) of them) at offsets R_T*64*hh.  Word index inside a
    half-block is ((q*R_T + j)*G_h + (g-2hh))*2 + u//2; the code of the weight
    sits at bits (pos, pos+1) with pos = 16*(e%2) + 14 - 2*(4*(u%2) + e//2),
    low code bit at pos.
tq5: each row's K trits are cut into segments of 640 (5 groups) plus a tail
    segment of L = K mod 640 trits.  A segment of L trits uses B = ceil(L/5)
    bytes (B = 128 for a full one); byte b of a segment holds the trits at
    segment offsets b + B*i, i = 0..4 (digit i); offsets >= L are padding
    trits 0 (digit 1).  Rows hold ceil(K/5) bytes.  Tile T starts at byte
    T*16*ceil(K/5); full segment S of tile T starts at R_T*128*S inside the
    tile and is laid out like a tq2 chunk: two half-blocks of R_T*64 bytes,
    byte ((q*R_T + j)*16 + w%16) of half-block w//16, where w = 8u + e and
    (u, q, e) come from b as above.  The tail segment of a tile is row-major:
    row j at R_T*128*S_full + j*B_tail.
Plane B (FP16 values, index = 2-byte slot after plane A): the scales follow
the units that read them.  Tile T holds the R_T*G scales of its rows from
index 16*T*G on; inside it the groups are cut into chunks of W (W = 4 for q1
and tq2, the chunks of plane A; W = 5 for tq5, its 640-trit segments), chunk
c (G_c = min(W, G-W*c) groups) starts at R_T*W*c inside the tile and holds
row j's G_c scales at j*G_c.  So the scale of (n, g) sits at
    16*T*G + R_T*W*c + j*G_c + (g - W*c),   c = g // W,
and the scales one unit (16 rows x one chunk) needs are contiguous.
"""
from __future__ import annotations

import numpy as np

GROUP = 128
FORMATS = ("q1", "tq2", "tq5")


def n_groups(K: int) -> int:
    if K % GROUP:
        raise ValueError("K must be a multiple of 128")
    return K // GROUP


def plane_a_bytes(fmt: str, N: int, K: int) -> int:
    if fmt == "q1":
        return N * K // 8
    if fmt == "tq2":
        return N * K // 4
    if fmt == "tq5":
        return N * (-(-K // 5))
    raise ValueError(fmt)


def packed_bytes(fmt: str, N: int, K: int) -> int:
    """Plane A plus one 2-byte scale per (row, group)."""
    return plane_a_bytes(fmt, N, K) + N * n_groups(K) * 2


# --------------------------------------------------------- address maps ----
def _tile(n, N):
    T = n // 16
    return T, n % 16, np.minimum(16, N - 16 * T)


def _in_group(k):
    kk = k % GROUP
    return kk // 32, (kk // 8) % 4, kk % 8


def q1_bit_index(n, k, N: int, K: int):
    """Bit index (byte*8 + bit) in plane A of the sign of weight (n, k)."""
    G = n_groups(K)
    T, j, R = _tile(n, N)
    ga = k // GROUP
    c, g = ga // 4, ga % 4
    Gc = np.minimum(4, G - 4 * c)
    u, q, e = _in_group(k)
    block = 16 * T * G * 16 + R * 4 * c * 16
    word = (q * R + j) * Gc + g
    pos = 16 * (e % 2) + 15 - ((e // 2) % 2) - 2 * (2 * u + (e // 2) // 2)
    return (block + 4 * word) * 8 + pos


def tq2_bit_index(n, k, N: int, K: int):
    """Bit index of the low bit of the 2-bit code of weight (n, k)."""
    G = n_groups(K)
    T, j, R = _tile(n, N)
    ga = k // GROUP
    c, g = ga // 4, ga % 4
    Gc = np.minimum(4, G - 4 * c)
    u, q, e = _in_group(k)
    hh = g // 2
    Gh = np.minimum(2, Gc - 2 * hh)
    block = 16 * T * G * 32 + R * 4 * c * 32 + R * 64 * hh
    word = ((q * R + j) * Gh + (g - 2 * hh)) * 2 + u // 2
    pos = 16 * (e % 2) + 14 - 2 * (4 * (u % 2) + e // 2)
    return (block + 4 * word) * 8 + pos


def tq5_geometry(K: int):
    s_full = K // 640
    L_tail = K - 640 * s_full
    b_tail = -(-L_tail // 5)
    return s_full, L_tail, b_tail, 128 * s_full + b_tail


def tq5_byte_digit(n, k, N: int, K: int):
    """(byte offset in plane A, base-3 digit index) of weight (n, k)."""
    s_full, L_tail, b_tail, rowbytes = tq5_geometry(K)
    T, j, R = _tile(n, N)
    S = k // 640
    full = S < s_full
    # full segment
    kseg = k - 640 * S
    i_full, b = kseg // 128, kseg % 128
    u, q, e = b // 32, (b // 8) % 4, b % 8
    w = 8 * u + e
    off_full = 16 * T * rowbytes + R * 128 * S + R * 64 * (w // 16) + (q * R + j) * 16 + w % 16
    # tail segment
    kt = k - 640 * s_full
    bt = max(b_tail, 1)
    i_tail, b_t = kt // bt, kt % bt
    off_tail = 16 * T * rowbytes + R * 128 * s_full + j * b_tail + b_t
    return np.where(full, off_full, off_tail), np.where(full, i_full, i_tail)


def scale_chunk_groups(fmt: str) -> int:
    return 5 if fmt == "tq5" else 4


def scale_index(fmt: str, n, g, N: int, K: int):
    """Index (in FP16 values) in plane B of the scale of row n, group g."""
    G = n_groups(K)
    W = scale_chunk_groups(fmt)
    T, j, R = _tile(n, N)
    c = g // W
    Gc = np.minimum(W, G - W * c)
    return 16 * T * G + R * W * c + j * Gc + (g - W * c)


# ----------------------------------------------------------- pack/unpack ----
def _row_blocks(N: int, rows_per_block: int = 1024):
    step = max(16, rows_per_block - rows_per_block % 16)
    for n0 in range(0, N, step):
        yield n0, min(N, n0 + step)


def pack(fmt: str, codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """codes int8[N,K], scales uint16[N,K/128] -> uint8 blob of packed_bytes()."""
    codes = np.asarray(codes)
    N, K = codes.shape
    G = n_groups(K)
    scales = np.asarray(scales, dtype=np.uint16).reshape(N, G)
    allowed = (-1, 1) if fmt == "q1" else (-1, 0, 1)
    if not np.isin(codes, allowed).all():
        raise ValueError("code outside the format's value set")
    a_bytes = plane_a_bytes(fmt, N, K)
    plane = np.zeros(a_bytes, dtype=np.uint8)
    kk = np.arange(K, dtype=np.int64)[None, :]
    if fmt in ("q1", "tq2"):
        bits = np.zeros(a_bytes * 8, dtype=np.uint8)
        for n0, n1 in _row_blocks(N):
            nn = np.arange(n0, n1, dtype=np.int64)[:, None]
            cb = codes[n0:n1]
            if fmt == "q1":
                idx = q1_bit_index(nn, kk, N, K)
                bits[idx] = (cb == 1)
            else:
                idx = tq2_bit_index(nn, kk, N, K)
                c = (cb.astype(np.int16) + 1).astype(np.uint8)
                bits[idx] = c & 1
                bits[idx + 1] = c >> 1
        plane[:] = np.packbits(bits, bitorder="little")
    else:
        # Every byte starts as all digits 1 (= all trits 0, value 1+3+9+27+81);
        # each weight then adds t * 3^i at its (byte, digit), since d = t + 1.
        val = np.full(a_bytes, 1 + 3 + 9 + 27 + 81, dtype=np.int64)
        for n0, n1 in _row_blocks(N):
            nn = np.arange(n0, n1, dtype=np.int64)[:, None]
            off, dig = tq5_byte_digit(nn, kk, N, K)
            contrib = codes[n0:n1].astype(np.int64) * (3 ** dig)
            lo = int(off.min())
            acc = np.bincount((off - lo).ravel(), weights=contrib.ravel().astype(np.float64))
            val[lo:lo + acc.size] += np.rint(acc).astype(np.int64)
        plane[:] = val.astype(np.uint8)
    sc_plane = np.zeros(N * G, dtype=np.uint16)
    gg = np.arange(G, dtype=np.int64)[None, :]
    for n0, n1 in _row_blocks(N):
        nn = np.arange(n0, n1, dtype=np.int64)[:, None]
        sc_plane[scale_index(fmt, nn, gg, N, K)] = scales[n0:n1]
    return np.concatenate([plane, sc_plane.view(np.uint8)])


class FormatError(ValueError):
    pass


def unpack(fmt: str, blob, N: int, K: int, rows=None):
    """Inverse of pack: (codes int8[len(rows),K], scales uint16[len(rows),G]).

    Raises FormatError on a tq2 code 3, a tq5 byte >= 243, or a tq5 padding
    trit that is not 0.  ``rows`` selects a subset of rows (default: all).
    """
    blob = np.asarray(blob, dtype=np.uint8).reshape(-1)
    G = n_groups(K)
    if blob.size < packed_bytes(fmt, N, K):
        raise FormatError("blob shorter than packed_bytes")
    rows = np.arange(N, dtype=np.int64) if rows is None else np.asarray(rows, dtype=np.int64)
    a_bytes = plane_a_bytes(fmt, N, K)
    sc_plane = blob[a_bytes:a_bytes + N * G * 2].view(np.uint16)
    sc = sc_plane[scale_index(fmt, rows[:, None], np.arange(G, dtype=np.int64)[None, :], N, K)]
    codes = np.zeros((rows.size, K), dtype=np.int8)
    kk = np.arange(K, dtype=np.int64)[None, :]
    for r0 in range(0, rows.size, 1024):
        nn = rows[r0:r0 + 1024, None]
        if fmt == "q1":
            idx = q1_bit_index(nn, kk, N, K)
            bit = (blob[idx // 8] >> (idx % 8)) & 1
            codes[r0:r0 + 1024] = np.where(bit == 1, 1, -1)
        elif fmt == "tq2":
            idx = tq2_bit_index(nn, kk, N, K)
            c = ((blob[idx // 8] >> (idx % 8)) & 3).astype(np.int16)
            if (c == 3).any():
                raise FormatError("tq2 code 3")
            codes[r0:r0 + 1024] = c - 1
        else:
            off, dig = tq5_byte_digit(nn, kk, N, K)
            v = blob[off].astype(np.int64)
            if (v >= 243).any():
                raise FormatError("tq5 byte >= 243")
            codes[r0:r0 + 1024] = (v // (3 ** dig)) % 3 - 1
    if fmt == "tq5":
        _check_tq5_padding(blob, N, K, rows)
    return codes, sc


def _check_tq5_padding(blob, N, K, rows):
    s_full, L_tail, b_tail, rowbytes = tq5_geometry(K)
    if b_tail == 0:
        return
    plane = blob[: plane_a_bytes("tq5", N, K)]
    for n in rows:
        T, j = n // 16, n % 16
        R = min(16, N - 16 * T)
        base = 16 * T * rowbytes + R * 128 * s_full + j * b_tail
        for b in range(b_tail):
            v = int(plane[base + b])
            if v >= 243:
                raise FormatError("tq5 byte >= 243")
            for i in range(5):
                if b + b_tail * i >= L_tail and (v // 3 ** i) % 3 != 1:
                    raise FormatError("tq5 padding trit is not 0")
