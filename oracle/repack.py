"""Reference implementation of the repacked INT4 tile layout (test infrastructure only).

The layout is this library's own (the pages give none); it is written out here
independently of the device code so that the device repack can be checked byte
for byte, and so that ``unrepack_ref(repack_ref(.))`` pins it as a bijection.
The point of repacking once, offline, is the one [P5] "关键数据解读" item 4
makes: a format whose layout is translated on every run is slow.

Layout (K tiles of 128 inputs, KT = K / 128, NP = ceil(N / 64); group size G
in {32, 64} or a multiple of 128 that divides K, G = K being per-channel):

* Column permutation.  If ``g_idx`` is given and is not the trivial
  k // G map, ``perm`` = stable argsort(g_idx): permuted column k' is original
  column perm[k'], and every run of G permuted columns is one whole group
  (act-order, [P2] §三 3.1 / [P4] "技术原理" section).  Otherwise perm is None.
* Codes: uint8 [NP][KT][4][64][16].  For output column n = 64p + 16c + i and
  permuted column k' = 128t + 32j + 8b + e, the code sits in lane l = i + 16b,
  32-bit word j of that lane's 16 bytes (little endian), at nibble slot
  (e >> 1) + 4 * (e & 1).  Columns n >= N are zero padding.
* Meta units: U = 128 / G units per K tile when G < 128 (unit u of tile t
  covers permuted columns 128t + uG ..; word j of a lane lies in unit
  jU / 4), else U = 1 and the unit of tile t carries the scale and zero of the
  group holding columns 128t .. 128t + 127 (repeated on each tile of a group
  that spans several).  Units are numbered v = tU + u.
* Scales, in runs of 8 tiles (KT8 = ceil(KT / 8)): fp16 [NP][KT8][4][16][8U],
  entry [p][g][c][i][r] = scale of column 64p + 16c + i in unit 8Ug + r
  (0 for padding columns and for units past the last tile).
* Zeros: uint32 [NP][KT8][4][16][U], bits [4e, 4e + 4) of word w of
  [p][g][c][i] = zero of column 64p + 16c + i in unit 8Ug + 8w + e (0 for
  padding).  A symmetric weight (no zeros) has no zeros array.
"""

import numpy as np

from .int4 import unpack_qweight, unpack_qzeros, default_g_idx

GROUP = 128
TILE = 128


def nibble_slot(e):
    return (e >> 1) + 4 * (e & 1)


def valid_group_size(K, G):
    return K % TILE == 0 and (G in (32, 64) or (G > 0 and G % TILE == 0 and K % G == 0))


def units_per_tile(G):
    return TILE // G if G < TILE else 1


def unit_groups(K, G):
    """Group (in permuted column order) of every meta unit v = t U + u."""
    U, KT = units_per_tile(G), K // TILE
    t = np.arange(KT)[:, None]
    u = np.arange(U)[None, :]
    return ((TILE * t + u * min(G, TILE)) // G).reshape(-1)


def canonical_perm(g_idx, K, group_size=GROUP):
    """perm for a g_idx, or None when g_idx is absent or trivial."""
    if g_idx is None:
        return None
    gi = np.asarray(g_idx, dtype=np.int64)
    if np.array_equal(gi, default_g_idx(K, group_size)):
        return None
    return np.argsort(gi, kind="stable").astype(np.int32)


def repack_ref(qweight, scales, qzeros, g_idx=None, group_size=GROUP):
    """Canonical GPTQ-style tensors -> (codes_r, scales_r, zeros_r, perm).

    ``qzeros=None`` (symmetric) gives zeros_r = None."""
    G = int(group_size)
    q = unpack_qweight(qweight)                      # [N, K]
    N, K = q.shape
    assert valid_group_size(K, G)
    s = np.asarray(scales, dtype=np.float16)         # [K/G, N]
    z = None if qzeros is None else unpack_qzeros(qzeros)[:, :N]
    KT = K // TILE
    U = units_per_tile(G)
    NP = (N + 63) // 64
    perm = canonical_perm(g_idx, K, G)
    if perm is not None:
        q = q[:, perm]
    Np = NP * 64
    qp = np.zeros((Np, K), dtype=np.uint8)
    qp[:N] = q

    # qp[n, k'] with n = 64p + 16c + i and k' = 128t + 32j + 8b + e
    v = qp.reshape(NP, 4, 16, KT, 4, 4, 8).astype(np.uint32)   # p c i t j b e
    words = np.zeros((NP, 4, 16, KT, 4, 4), dtype=np.uint32)   # p c i t j b
    for e in range(8):
        words |= v[..., e] << np.uint32(4 * nibble_slot(e))
    # -> [p][t][c][lane = i + 16 b][j]
    words = words.transpose(0, 3, 1, 5, 2, 4).reshape(NP, KT, 4, 64, 4)
    codes_r = np.ascontiguousarray(words).view(np.uint8).reshape(-1)

    KT8 = (KT + 7) // 8
    V8 = KT8 * 8 * U                                  # units incl. the last run's padding
    ug = unit_groups(K, G)                            # [KT * U]
    su = np.zeros((V8, Np), dtype=np.float16)
    su[:KT * U, :N] = s[ug]
    # [g r][p c i] -> [p][g][c][i][r]
    scales_r = su.reshape(KT8, 8 * U, NP, 4, 16).transpose(2, 0, 3, 4, 1).copy().reshape(-1)
    zeros_r = None
    if z is not None:
        zu = np.zeros((V8, Np), dtype=np.uint32)
        zu[:KT * U, :N] = z[ug]
        zz = zu.reshape(KT8, U, 8, NP, 4, 16).transpose(3, 0, 4, 5, 1, 2)   # p g c i w e
        zr = np.zeros((NP, KT8, 4, 16, U), dtype=np.uint32)
        for e in range(8):
            zr |= zz[..., e] << np.uint32(4 * e)
        zeros_r = zr.reshape(-1)
    return codes_r, scales_r, zeros_r, perm


def unrepack_ref(codes_r, scales_r, zeros_r, K, N, group_size=GROUP):
    """Inverse of the tile layout: -> (codes [N, K] in permuted column order,
    scales fp16 [K/G, N], zeros uint8 [K/G, N] or None).  Raises if the units
    of one group disagree."""
    G = int(group_size)
    KT = K // TILE
    U = units_per_tile(G)
    NP = (N + 63) // 64
    words = np.asarray(codes_r, dtype=np.uint8).view(np.uint32).reshape(NP, KT, 4, 4, 16, 4)
    # p t c b i j -> p c i t j b
    words = words.transpose(0, 2, 4, 1, 5, 3)
    v = np.zeros(words.shape + (8,), dtype=np.uint8)
    for e in range(8):
        v[..., e] = (words >> np.uint32(4 * nibble_slot(e))) & np.uint32(0xF)
    q = v.reshape(NP * 64, K)[:N]
    KT8 = (KT + 7) // 8
    ug = unit_groups(K, G)

    def from_units(units):                           # [KT * U, N] -> [K / G, N]
        out = units[np.searchsorted(ug, np.arange(K // G))]
        if not np.array_equal(units, out[ug]):
            raise ValueError("meta units of one group disagree")
        return out

    su = np.asarray(scales_r, dtype=np.float16).reshape(NP, KT8, 4, 16, 8 * U)
    su = su.transpose(1, 4, 0, 2, 3).reshape(KT8 * 8 * U, NP * 64)[:KT * U, :N]
    s = from_units(su)
    z = None
    if zeros_r is not None:
        zr = np.asarray(zeros_r, dtype=np.uint32).reshape(NP, KT8, 4, 16, U)
        z8 = np.zeros((NP, KT8, 4, 16, U, 8), dtype=np.uint8)
        for e in range(8):
            z8[..., e] = (zr >> np.uint32(4 * e)) & np.uint32(0xF)
        zu = z8.transpose(1, 4, 5, 0, 2, 3).reshape(KT8 * 8 * U, NP * 64)[:KT * U, :N]
        z = from_units(zu)
    return q.copy(), s.copy(), None if z is None else z.copy()


# --------------------------------------------------- 3- and 8-bit tile layouts
#
# The same tiles (16 columns x 128 permuted inputs, lane l = i + 16b holding
# inputs 128t + 32j + 8b + e of column i for the 4 MFMA steps j), with the
# lane's 32 codes in b-bit form:
#
# * b = 4: as above (4 dwords, dword j, nibble slot (e >> 1) + 4(e & 1)).
# * b = 8: 8 dwords per lane in two halves h = j >> 1 of 16 bytes each; the
#   tile is uint8 [2][64][16] (so each half of the tile is 1 KB contiguous).
#   Code (j, e) sits in dword 2(j & 1) + (e >> 2) of half j >> 1, at byte slot
#   ((e & 3) >> 1) + 2(e & 1): a dword holds elements [e0, e2, e1, e3] so that
#   (d >> 8r) & 0x00FF00FF is the element pair (2r, 2r + 1).
# * b = 3: 3 dwords per lane (tile uint8 [64][12]).  The low 2 bits of code
#   (j, e) sit in dword j >> 1 at bit 16(e & 1) + 2(4(j & 1) + (e >> 1)); its
#   high bit in dword 2 at bit 16(e & 1) + 4j + (e >> 1).
#
# Zeros: 4-bit fields (b <= 4, as above) or 8-bit fields (b = 8: U x 2 dwords
# per (panel, run, column), unit r of the run at byte r).  Scales as above.

TILE_DWORDS = {3: 3, 4: 4, 8: 8}


def _code_parts(bits, j, e):
    """[(dword index within the lane's tile dwords, bit shift, value bits)]
    for code (j, e): value bits = (mask, right shift) applied to the code."""
    if bits == 4:
        return [(j, 4 * nibble_slot(e), (0xF, 0))]
    if bits == 8:
        return [(4 * (j >> 1) + 2 * (j & 1) + (e >> 2), 8 * (((e & 3) >> 1) + 2 * (e & 1)),
                 (0xFF, 0))]
    return [(j >> 1, 16 * (e & 1) + 2 * (4 * (j & 1) + (e >> 1)), (0x3, 0)),
            (2, 16 * (e & 1) + 4 * j + (e >> 1), (0x1, 2))]


def _lane_dwords_to_bytes(words, bits):
    """words [NP, KT, 4, 64, D] -> the tile byte order of ``bits``."""
    if bits == 8:   # [.., 64, 2 halves, 4] -> [.., 2, 64, 4]
        words = words.reshape(words.shape[:-1] + (2, 4)).swapaxes(-3, -2)
    return np.ascontiguousarray(words).view(np.uint8).reshape(-1)


def _bytes_to_lane_dwords(codes_r, bits, NP, KT):
    D = TILE_DWORDS[bits]
    w = np.asarray(codes_r, dtype=np.uint8).view(np.uint32)
    if bits == 8:
        return w.reshape(NP, KT, 4, 2, 64, 4).swapaxes(-3, -2).reshape(NP, KT, 4, 64, 8)
    return w.reshape(NP, KT, 4, 64, D)


def repack_ref_bits(qweight, scales, qzeros, bits, g_idx=None, group_size=GROUP):
    """b-bit canonical tensors (``intb`` packing) -> (codes_r, scales_r, zeros_r, perm)."""
    from .intb import unpack_qweight as unpack_b, unpack_qzeros as unpack_zb
    G = int(group_size)
    q = unpack_b(qweight, bits)
    N, K = q.shape
    assert valid_group_size(K, G)
    s = np.asarray(scales, dtype=np.float16)
    z = None if qzeros is None else unpack_zb(qzeros, bits)[:, :N]
    KT, U, NP = K // TILE, units_per_tile(G), (N + 63) // 64
    perm = canonical_perm(g_idx, K, G)
    if perm is not None:
        q = q[:, perm]
    Np = NP * 64
    qp = np.zeros((Np, K), dtype=np.uint8)
    qp[:N] = q
    v = qp.reshape(NP, 4, 16, KT, 4, 4, 8).astype(np.uint32)        # p c i t j b e
    words = np.zeros((NP, KT, 4, 4, 16, TILE_DWORDS[bits]), dtype=np.uint32)  # p t c b i d
    for j in range(4):
        for e in range(8):
            code = v[:, :, :, :, j, :, e].transpose(0, 3, 1, 4, 2)     # p t c b i
            for d, sh, (mask, rs) in _code_parts(bits, j, e):
                words[..., d] |= ((code >> np.uint32(rs)) & np.uint32(mask)) << np.uint32(sh)
    codes_r = _lane_dwords_to_bytes(words.reshape(NP, KT, 4, 64, TILE_DWORDS[bits]), bits)

    KT8 = (KT + 7) // 8
    V8 = KT8 * 8 * U
    ug = unit_groups(K, G)
    su = np.zeros((V8, Np), dtype=np.float16)
    su[:KT * U, :N] = s[ug]
    scales_r = su.reshape(KT8, 8 * U, NP, 4, 16).transpose(2, 0, 3, 4, 1).copy().reshape(-1)
    zeros_r = None
    if z is not None:
        zu = np.zeros((V8, Np), dtype=np.uint32)
        zu[:KT * U, :N] = z[ug]
        per, width = (4, 8) if bits == 8 else (8, 4)                  # fields per dword, bits
        nw = 8 * U // per
        zz = zu.reshape(KT8, nw, per, NP, 4, 16).transpose(3, 0, 4, 5, 1, 2)   # p g c i w f
        zr = np.zeros((NP, KT8, 4, 16, nw), dtype=np.uint32)
        for f in range(per):
            zr |= zz[..., f] << np.uint32(width * f)
        zeros_r = zr.reshape(-1)
    return codes_r, scales_r, zeros_r, perm


def unrepack_ref_bits(codes_r, scales_r, zeros_r, K, N, bits, group_size=GROUP):
    """Inverse of repack_ref_bits: (codes [N, K] permuted order, scales [K/G, N],
    zeros [K/G, N] or None)."""
    G = int(group_size)
    KT, U, NP = K // TILE, units_per_tile(G), (N + 63) // 64
    words = _bytes_to_lane_dwords(codes_r, bits, NP, KT).reshape(NP, KT, 4, 4, 16, -1)
    v = np.zeros((NP, 4, 16, KT, 4, 4, 8), dtype=np.uint8)            # p c i t j b e
    for j in range(4):
        for e in range(8):
            code = np.zeros((NP, KT, 4, 4, 16), dtype=np.uint32)
            for d, sh, (mask, rs) in _code_parts(bits, j, e):
                code |= ((words[..., d] >> np.uint32(sh)) & np.uint32(mask)) << np.uint32(rs)
            v[:, :, :, :, j, :, e] = code.transpose(0, 2, 4, 1, 3)
    q = v.reshape(NP * 64, K)[:N]
    KT8 = (KT + 7) // 8
    ug = unit_groups(K, G)

    def from_units(units):
        out = units[np.searchsorted(ug, np.arange(K // G))]
        if not np.array_equal(units, out[ug]):
            raise ValueError("meta units of one group disagree")
        return out

    su = np.asarray(scales_r, dtype=np.float16).reshape(NP, KT8, 4, 16, 8 * U)
    s = from_units(su.transpose(1, 4, 0, 2, 3).reshape(KT8 * 8 * U, NP * 64)[:KT * U, :N])
    z = None
    if zeros_r is not None:
        per, width = (4, 8) if bits == 8 else (8, 4)
        nw = 8 * U // per
        zr = np.asarray(zeros_r, dtype=np.uint32).reshape(NP, KT8, 4, 16, nw)
        zf = np.zeros((NP, KT8, 4, 16, nw, per), dtype=np.uint8)
        for f in range(per):
            zf[..., f] = (zr >> np.uint32(width * f)) & np.uint32((1 << width) - 1)
        zu = zf.transpose(1, 4, 5, 0, 2, 3).reshape(KT8 * 8 * U, NP * 64)[:KT * U, :N]
        z = from_units(zu)
    return q.copy(), s.copy(), z


# ---- NF4 codes in the same 1 KB tiles (test infrastructure only).
#
# NF4 weights keep their canonical scales (absmax_q, absmax_scale); only the
# codes are re-laid, once, into tiles of 16 output rows x 128 inputs, so that a
# wavefront reads a tile as one contiguous 1 KB block instead of 16 rows of
# 64 bytes at the row pitch (the point of [P5] "关键数据解读" item 4: layout is
# translated once, offline, never per run).  With KT = ceil(K / 128):
#
# * codes_r uint8 [N / 16][KT][64][16]; entry [c][t][l][j] is byte
#   64 t + 16 (l >> 4) + j of canonical row 16 c + (l & 15) (that row's codes
#   of inputs 128 t + 32 (l >> 4) + 2 j and + 1, low nibble first), 0 past the
#   row's K / 2 bytes.

def repack_nf4_ref(qweight, N, K):
    """qweight uint8 [N, K/2] (canonical NF4 packing) -> codes_r (flat uint8)."""
    assert N % 16 == 0 and K % 64 == 0
    KT = (K + TILE - 1) // TILE
    rows_bytes = K // 2
    out = np.zeros((N // 16, KT, 64, 16), dtype=np.uint8)
    for c in range(N // 16):
        for t in range(KT):
            for l in range(64):
                row = 16 * c + (l & 15)
                b0 = 64 * t + 16 * (l >> 4)
                for j in range(16):
                    if b0 + j < rows_bytes:
                        out[c, t, l, j] = qweight[row, b0 + j]
    return out.reshape(-1)


def unrepack_nf4_ref(codes_r, N, K):
    """The inverse: codes_r -> canonical qweight uint8 [N, K/2]."""
    KT = (K + TILE - 1) // TILE
    r = np.asarray(codes_r, dtype=np.uint8).reshape(N // 16, KT, 64, 16)
    q = np.zeros((N, K // 2), dtype=np.uint8)
    for c in range(N // 16):
        for t in range(KT):
            for l in range(64):
                row = 16 * c + (l & 15)
                b0 = 64 * t + 16 * (l >> 4)
                for j in range(16):
                    if b0 + j < K // 2:
                        q[row, b0 + j] = r[c, t, l, j]
    return q
