"""b-bit (3, 4 or 8) group-wise integer weights: quantizer, packing, dequant.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix, restated: besides the 4-bit default, weight-only
quantization is used at 8 bits (small loss, small saving) and at 3 bits
(more saving, visible quality loss) ([P3] §2.3; the GPTQ-3bit and AWQ-3bit
rows of the [P1] §4.1 table; [P4] "量化效果PK" on 3-bit codes with groups of
128, and "部署实战" on the bit-width option of 4 or 8).  The method is the same as at 4 bits: a
scale (and, for asymmetric codes, a zero) per group of G inputs of an output
channel, codes in [0, 2^b - 1].

Readings taken where the pages are silent:
* Quantizer: the 4-bit one of ``int4.py`` with 2^b - 1 levels.
  Asymmetric: s = fp16(fp32(max - min) / (2^b - 1)), z = clip(rint(-min / s),
  0, 2^b - 1), q = clip(rint(w / s) + z, 0, 2^b - 1).  Symmetric: s =
  fp16(fp32(max |w|) / (2^(b-1) - 1)), q = clip(rint(w / s), -2^(b-1),
  2^(b-1) - 1) + 2^(b-1), no zeros (implicit zero 2^(b-1)).  A group whose
  fp16 scale is 0 uses s = 1.  Decisions in fp32, rint half to even.
* Packing, GPTQ style, in the ORIGINAL column order: along K for ``qweight``
  int32 [K b / 32, N] and along N for ``qzeros`` int32 [K/G, N b / 32].  Each
  run of 32 consecutive codes is one little-endian bit stream of b * 32 bits
  (b words): code e at bits [b e, b e + b).  At b = 4 and 8 no code crosses a
  word (the stream is also whole words every 8 or 4 codes, so N need only be
  a multiple of 8 or 4 for the zeros); at b = 3 codes 10 and 21 do, and N is a
  multiple of 32.
* Dequant: w = round16(fp32(q - z) * fp32(s)) with the product exact in fp32
  (a 9-bit integer times an 11-bit significand at most).
"""

import numpy as np

from .fp import round_to

BITS = (3, 4, 8)


def sym_zero(bits):
    return 1 << (bits - 1)


def default_g_idx(K, group_size):
    return (np.arange(K, dtype=np.int64) // group_size).astype(np.int32)


def quantize_rtn(W, bits, group_size=128, g_idx=None, sym=False):
    """RTN-quantize W [N, K] fp32 -> (q uint8 [N, K], scales fp16 [K/G, N],
    zeros uint8 [K/G, N] or None when symmetric)."""
    assert bits in BITS
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    G = int(group_size)
    assert K % G == 0
    ng = K // G
    qmax = (1 << bits) - 1
    half = sym_zero(bits)
    gi = default_g_idx(K, G) if g_idx is None else np.asarray(g_idx, dtype=np.int64)
    q = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((ng, N), dtype=np.float16)
    zeros = None if sym else np.zeros((ng, N), dtype=np.uint8)
    for g in range(ng):
        cols = np.nonzero(gi == g)[0]
        Wg = W[:, cols]
        if sym:
            s32 = np.abs(Wg).max(axis=1) / np.float32(half - 1)
        else:
            mn = Wg.min(axis=1)
            s32 = (Wg.max(axis=1) - mn) / np.float32(qmax)
        s16 = s32.astype(np.float16)
        s16 = np.where(s16 == 0, np.float16(1.0), s16)
        sf = s16.astype(np.float32)
        if sym:
            c = np.clip(np.rint(Wg / sf[:, None]), -half, half - 1)
            q[:, cols] = (c + half).astype(np.uint8)
        else:
            z = np.clip(np.rint(-mn / sf), 0, qmax)
            q[:, cols] = np.clip(np.rint(Wg / sf[:, None]) + z[:, None], 0, qmax).astype(np.uint8)
            zeros[g] = z.astype(np.uint8)
        scales[g] = s16
    return q, scales, zeros


def run_codes(bits):
    """Codes per run of whole words: 32 / gcd(b, 32) (8 at b = 4, 4 at b = 8,
    32 at b = 3); the stream of a longer run of 32 is the same bits."""
    return 32 // int(np.gcd(bits, 32))


def _pack_runs(codes, bits):
    """codes [R, C] -> uint32 [R b / 32, C]: every run of L = run_codes(b) rows
    is a little-endian bit stream of L b / 32 words, code e at bits [b e, b e + b)."""
    codes = np.asarray(codes, dtype=np.uint64)
    R, C = codes.shape
    L = run_codes(bits)
    nw = L * bits // 32
    assert R % L == 0
    c = codes.reshape(R // L, L, C)
    out = np.zeros((R // L, nw, C), dtype=np.uint64)
    for e in range(L):
        pos = bits * e
        word, sh = pos // 32, pos % 32
        out[:, word] |= (c[:, e] << np.uint64(sh)) & np.uint64(0xFFFFFFFF)
        if sh + bits > 32:                             # the code continues in the next word
            out[:, word + 1] |= c[:, e] >> np.uint64(32 - sh)
    return out.astype(np.uint32).reshape(R // L * nw, C)


def _unpack_runs(words, bits):
    w = np.asarray(words).view(np.uint32).astype(np.uint64)
    Rw, C = w.shape
    L = run_codes(bits)
    nw = L * bits // 32
    assert Rw % nw == 0
    w = w.reshape(Rw // nw, nw, C)
    out = np.zeros((Rw // nw, L, C), dtype=np.uint8)
    mask = np.uint64((1 << bits) - 1)
    for e in range(L):
        pos = bits * e
        word, sh = pos // 32, pos % 32
        v = w[:, word] >> np.uint64(sh)
        if sh + bits > 32:
            v |= w[:, word + 1] << np.uint64(32 - sh)
        out[:, e] = (v & mask).astype(np.uint8)
    return out.reshape(Rw // nw * L, C)


def pack_qweight(q, bits):
    """Codes [N, K] -> int32 [K b / 32, N] (runs of 32 codes along K)."""
    return _pack_runs(np.asarray(q).T, bits).view(np.int32)


def unpack_qweight(qweight, bits):
    """int32 [K b / 32, N] -> codes uint8 [N, K]."""
    return _unpack_runs(qweight, bits).T.copy()


def pack_qzeros(z, bits):
    """Zeros [K/G, N] -> int32 [K/G, N b / 32] (runs of 32 zeros along N)."""
    return _pack_runs(np.asarray(z).T, bits).T.copy().view(np.int32)


def unpack_qzeros(qzeros, bits):
    """int32 [K/G, N b / 32] -> zeros uint8 [K/G, N]."""
    return _unpack_runs(np.asarray(qzeros).T, bits).T.copy()


def dequant_codes(q, scales, zeros, bits, g_idx=None, group_size=128, dtype="f16"):
    """w[n, k] = round_dtype(fp32(q - z) * fp32(s)), z = 2^(b-1) when zeros is None."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    s = np.asarray(scales, dtype=np.float16)
    z = (np.full(s.shape, sym_zero(bits), dtype=np.uint8) if zeros is None
         else np.asarray(zeros, dtype=np.uint8))
    gi = default_g_idx(K, group_size) if g_idx is None else np.asarray(g_idx, dtype=np.int64)
    zk = z[gi, :].T.astype(np.float32)
    sk = s[gi, :].T.astype(np.float32)
    return round_to((q.astype(np.float32) - zk) * sk, dtype)
