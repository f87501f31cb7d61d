"""NF4 (bitsandbytes-style) oracle: codebook, block quantizer, double quant, dequant.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix, restated:
* bitsandbytes quantizes weights block by block, each block with its own
  absolute-maximum statistic ([P1] §2.3; [P4] "技术原理" section);
* NF4 puts the 16 representable values at quantiles of a standard normal
  distribution, so they crowd around zero where LLM weights sit ([P1] §2.3 and
  §3.3; [P5] "关键数据解读" item 2);
* double quantization also quantizes the per-block scales, storing a
  "scale of the scale" ([P1] §4.3 pitfall 3; [P4] "技术原理" and "部署实战");
* the 4-bit codes are stored in uint8 tensors with a ``quant_state`` holding
  ``absmax`` ([P1] §3.3); bitsandbytes dequantizes to 16 bits on every forward
  ([P5] "关键数据解读" item 2).

[P1] §3.3 prints the level formula in a garbled form (endpoints -3/+3 and
Phi^-1(i/15), which diverges at i = 0).  The reading taken is the published NF4
construction: 8 positive levels at Phi^-1 of 8 equal steps from 1/2 to delta,
7 negative levels mirrored from 7 equal steps, one exact zero, everything
divided by Phi^-1(delta) so the range is [-1, 1], with
delta = ((1 - 1/30) + (1 - 1/32)) / 2.  Levels are rounded once to fp32.

Other readings taken where the pages are silent:
* a block is 64 consecutive elements of row-major W [N, K] (K % 64 == 0);
* code = argmin_i |w/absmax - L_i| with w/absmax and the distances in fp32;
  ties go to the lower index; an all-zero block gives code 7 (L_7 = 0);
* packing: uint8 [N, K/2], element 2j in the low nibble of byte j;
* double quant: groups of 256 consecutive blocks; absmax_scale =
  fp32(max absmax / 255); absmax_q = clip(rint(absmax / absmax_scale), 0, 255)
  (0 when the group scale is 0); codes use the exact fp32 absmax;
* dequant: a' = fp32(fp32(absmax_q) * absmax_scale[b // 256]);
  w = round16(fp32(L[c] * a')) for fp16 or bf16 output.
"""

from statistics import NormalDist

import numpy as np

from .fp import round_to

DQ_GROUP = 256


def nf4_delta():
    return 0.5 * ((1.0 - 1.0 / 30.0) + (1.0 - 1.0 / 32.0))


def nf4_codebook():
    """The 16 NF4 levels as fp32, ascending, L[0] = -1, L[7] = 0, L[15] = 1."""
    inv = NormalDist().inv_cdf
    d = nf4_delta()
    pos = [inv(p) for p in np.linspace(d, 0.5, 9)[:-1]]      # 8 positive levels
    neg = [-inv(p) for p in np.linspace(d, 0.5, 8)[:-1]]     # 7 negative levels
    vals = sorted(pos + [0.0] + neg)
    top = inv(d)
    return np.array([v / top for v in vals], dtype=np.float64).astype(np.float32)


def quantize_nf4(W, blocksize=64, codebook=None, rows_per_chunk=256):
    """Block-wise NF4 quantization of W [N, K] fp32.

    Returns (codes uint8 [N, K], absmax fp32 [N*K/blocksize]).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    assert K % blocksize == 0
    L = nf4_codebook() if codebook is None else np.asarray(codebook, dtype=np.float32)
    codes = np.zeros((N, K), dtype=np.uint8)
    absmax = np.zeros(N * K // blocksize, dtype=np.float32)
    bpr = K // blocksize
    for r0 in range(0, N, rows_per_chunk):
        r1 = min(N, r0 + rows_per_chunk)
        blk = W[r0:r1].reshape(-1, blocksize)
        am = np.abs(blk).max(axis=1)
        safe = np.where(am == 0, np.float32(1.0), am)
        v = np.where(am[:, None] == 0, np.float32(0.0), blk / safe[:, None])
        dist = np.abs(v[:, :, None] - L[None, None, :])     # fp32 distances
        c = np.argmin(dist, axis=2)                         # first minimum
        codes[r0:r1] = c.reshape(r1 - r0, K).astype(np.uint8)
        absmax[r0 * bpr:r1 * bpr] = am
    return codes, absmax


def double_quant(absmax, group=DQ_GROUP):
    """8-bit quantization of the block absmax values, one fp32 scale per group."""
    absmax = np.asarray(absmax, dtype=np.float32)
    nb = absmax.shape[0]
    ngr = (nb + group - 1) // group
    aq = np.zeros(nb, dtype=np.uint8)
    sc = np.zeros(ngr, dtype=np.float32)
    for g in range(ngr):
        a = absmax[g * group:(g + 1) * group]
        s = np.float32(a.max()) / np.float32(255.0)
        sc[g] = s
        if s > 0:
            aq[g * group:(g + 1) * group] = np.clip(np.rint(a / s), 0, 255).astype(np.uint8)
    return aq, sc


def pack_nf4(codes):
    """codes uint8 [N, K] -> uint8 [N, K/2]; element 2j low nibble of byte j."""
    c = np.asarray(codes, dtype=np.uint8)
    return (c[:, 0::2] | (c[:, 1::2] << 4)).astype(np.uint8)


def unpack_nf4(packed):
    p = np.asarray(packed, dtype=np.uint8)
    N, K2 = p.shape
    out = np.zeros((N, 2 * K2), dtype=np.uint8)
    out[:, 0::2] = p & 0xF
    out[:, 1::2] = p >> 4
    return out


def dequant_absmax(absmax_q, absmax_scale, group=DQ_GROUP):
    aq = np.asarray(absmax_q, dtype=np.uint8).astype(np.float32)
    sc = np.asarray(absmax_scale, dtype=np.float32)
    idx = np.arange(aq.shape[0]) // group
    return (aq * sc[idx]).astype(np.float32)


def dequant_nf4(qweight, absmax_q, absmax_scale, blocksize=64, dtype="bf16",
                codebook=None, rows=None):
    """Dequantize NF4 to uint16 bits of ``dtype``; optional subset of rows."""
    L = nf4_codebook() if codebook is None else np.asarray(codebook, dtype=np.float32)
    p = np.asarray(qweight, dtype=np.uint8)
    N, K2 = p.shape
    K = 2 * K2
    bpr = K // blocksize
    a = dequant_absmax(absmax_q, absmax_scale)
    rows = np.arange(N) if rows is None else np.asarray(rows)
    c = unpack_nf4(p[rows])                                  # [R, K]
    blk = rows[:, None] * bpr + (np.arange(K)[None, :] // blocksize)
    w32 = (L[c] * a[blk]).astype(np.float32)                 # one fp32 rounding
    return round_to(w32, dtype)
