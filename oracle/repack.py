"""Reference implementation of the repacked INT4 tile layout (test infrastructure only).

The layout is this library's own (the pages give none); it is written out here
independently of the device code so that the device repack can be checked byte
for byte, and so that ``unrepack_ref(repack_ref(.))`` pins it as a bijection.
The point of repacking once, offline, is the one [P5] "关键数据解读" item 4
makes: a format whose layout is translated on every run is slow.

Layout (G = 128, KT = K / G, NP = ceil(N / 64)):

* Column permutation.  If ``g_idx`` is given and is not the trivial
  k // G map, ``perm`` = stable argsort(g_idx): permuted column k' is original
  column perm[k'], and every run of G permuted columns is one whole group
  (act-order, [P2] §三 3.1 / [P4] "技术原理" section).  Otherwise perm is None.
* Codes: uint8 [NP][KT][4][64][16].  For output column n = 64p + 16c + i and
  permuted column k' = 128t + 32j + 8b + e, the code sits in lane l = i + 16b,
  32-bit word j of that lane's 16 bytes (little endian), at nibble slot
  (e >> 1) + 4 * (e & 1).  Columns n >= N are zero padding.
* Scales, in runs of 8 groups (KT8 = ceil(KT / 8)): fp16 [NP][KT8][4][16][8],
  entry [p][g][c][i][s] = scale of column 64p + 16c + i in group 8g + s
  (0 for padding columns and for groups >= KT).
* Zeros: uint32 [NP][KT8][4][16], bits [4s, 4s + 4) of [p][g][c][i] = zero
  of column 64p + 16c + i in group 8g + s (0 for padding).
"""

import numpy as np

from .int4 import unpack_qweight, unpack_qzeros, default_g_idx

GROUP = 128


def nibble_slot(e):
    return (e >> 1) + 4 * (e & 1)


def canonical_perm(g_idx, K, group_size=GROUP):
    """perm for a g_idx, or None when g_idx is absent or trivial."""
    if g_idx is None:
        return None
    gi = np.asarray(g_idx, dtype=np.int64)
    if np.array_equal(gi, default_g_idx(K, group_size)):
        return None
    return np.argsort(gi, kind="stable").astype(np.int32)


def repack_ref(qweight, scales, qzeros, g_idx=None, group_size=GROUP):
    """Canonical GPTQ-style tensors -> (codes_r, scales_r, zeros_r, perm)."""
    assert group_size == GROUP
    q = unpack_qweight(qweight)                      # [N, K]
    N, K = q.shape
    z = unpack_qzeros(qzeros)[:, :N]                 # [KT, N]
    s = np.asarray(scales, dtype=np.float16)         # [KT, N]
    KT = K // GROUP
    NP = (N + 63) // 64
    perm = canonical_perm(g_idx, K, group_size)
    if perm is not None:
        q = q[:, perm]
    Np = NP * 64
    qp = np.zeros((Np, K), dtype=np.uint8)
    qp[:N] = q
    zp = np.zeros((KT, Np), dtype=np.uint8)
    zp[:, :N] = z
    sp = np.zeros((KT, Np), dtype=np.float16)
    sp[:, :N] = s

    # qp[n, k'] with n = 64p + 16c + i and k' = 128t + 32j + 8b + e
    v = qp.reshape(NP, 4, 16, KT, 4, 4, 8).astype(np.uint32)   # p c i t j b e
    words = np.zeros((NP, 4, 16, KT, 4, 4), dtype=np.uint32)   # p c i t j b
    for e in range(8):
        words |= v[..., e] << np.uint32(4 * nibble_slot(e))
    # -> [p][t][c][lane = i + 16 b][j]
    words = words.transpose(0, 3, 1, 5, 2, 4).reshape(NP, KT, 4, 64, 4)
    codes_r = np.ascontiguousarray(words).view(np.uint8).reshape(-1)

    KT8 = (KT + 7) // 8
    sp8 = np.zeros((KT8 * 8, Np), dtype=np.float16)
    sp8[:KT] = sp
    zp8 = np.zeros((KT8 * 8, Np), dtype=np.uint32)
    zp8[:KT] = zp
    # [g s][p c i] -> [p][g][c][i][s]
    scales_r = sp8.reshape(KT8, 8, NP, 4, 16).transpose(2, 0, 3, 4, 1).copy()
    zz = zp8.reshape(KT8, 8, NP, 4, 16).transpose(2, 0, 3, 4, 1)          # p g c i s
    zeros_r = np.zeros((NP, KT8, 4, 16), dtype=np.uint32)
    for t8 in range(8):
        zeros_r |= zz[..., t8] << np.uint32(4 * t8)
    return codes_r, scales_r.reshape(-1), zeros_r.reshape(-1), perm


def unrepack_ref(codes_r, scales_r, zeros_r, K, N):
    """Inverse of the tile layout: -> (codes [N, K] in permuted column order,
    scales fp16 [KT, N], zeros uint8 [KT, N])."""
    KT = K // GROUP
    NP = (N + 63) // 64
    words = np.asarray(codes_r, dtype=np.uint8).view(np.uint32).reshape(NP, KT, 4, 4, 16, 4)
    # p t c b i j -> p c i t j b
    words = words.transpose(0, 2, 4, 1, 5, 3)
    v = np.zeros(words.shape + (8,), dtype=np.uint8)
    for e in range(8):
        v[..., e] = (words >> np.uint32(4 * nibble_slot(e))) & np.uint32(0xF)
    q = v.reshape(NP * 64, K)[:N]
    KT8 = (KT + 7) // 8
    s8 = np.asarray(scales_r, dtype=np.float16).reshape(NP, KT8, 4, 16, 8)
    s = s8.transpose(1, 4, 0, 2, 3).reshape(KT8 * 8, NP * 64)[:KT, :N]
    zr = np.asarray(zeros_r, dtype=np.uint32).reshape(NP, KT8, 4, 16)
    z8 = np.zeros((NP, KT8, 4, 16, 8), dtype=np.uint8)
    for t8 in range(8):
        z8[..., t8] = (zr >> np.uint32(4 * t8)) & np.uint32(0xF)
    z = z8.transpose(1, 4, 0, 2, 3).reshape(KT8 * 8, NP * 64)[:KT, :N]
    return q.copy(), s.copy(), z.copy()
