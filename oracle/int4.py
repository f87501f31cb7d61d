"""Group-wise INT4 (GPTQ/AWQ-style) oracle: quantizer, packing, dequant.

Test infrastructure only (see ``oracle/__init__.py``).

What the pages fix, restated:
* asymmetric quantization maps a float interval onto the integer interval and
  stores a zero point besides the scale ([P3] §2.1; [P2] §三 3.1 ``zero_point``);
* symmetric quantization maps the float interval symmetrically onto the
  integer interval with the zero point fixed at 0 ([P3] §2.1; AWQ's
  ``zero_point`` switch, [P3] §4.1 / [P2] §三 3.1);
* group-wise granularity: a run of G weights shares one scale, G = 128 by
  default and 64 or 32 for more accuracy at more bytes ([P3] §2.2, §3.1, §7.1;
  [P1] §3.1 node 3); per-channel granularity is one scale per output channel,
  i.e. G = K ([P3] §2.2);
* 4-bit codes, 16 levels ([P3] §2.3; [P2] §一);
* plain round-to-nearest (RTN) is the baseline quantizer GPTQ is compared with
  ([P4] "技术原理" section);
* act-order (``desc_act`` / ``--act-order``) quantizes columns in an
  importance order and records, for every input column, the group it fell in
  (``g_idx``) ([P2] §三 3.1; [P3] §3.1; [P4] "技术原理" section).

Readings taken where the pages are silent:
* W is [N, K] (row = output channel) and y = x W^T.
* Scale of a group: fp16 round of fp32((max - min) / 15); zero:
  clip(rint(-min / s), 0, 15); code: clip(rint(w / s) + z, 0, 15).  All code and
  zero decisions are taken in fp32 with the fp16 value of s (the precision the
  device kernels use); rint rounds half to even.  A group whose fp16 scale is 0
  (e.g. max == min) uses s = 1.
* Packing: ``qweight`` int32 [K/8, N]; bits [4j, 4j+4) of word (i, n) hold the
  code of (n, 8i + j) in the ORIGINAL column order.  ``qzeros`` int32
  [K/G, N/8]; bits [4j, 4j+4) of word (g, i) hold the zero of (g, 8i + j).
  The stored zero is the true zero (no offset).  ``scales`` fp16 [K/G, N].
* Symmetric reading: the signed code c = clip(rint(w / s), -8, 7) with
  s = fp16 round of fp32(max |w| / 7) (so +-max|w| map to +-7, the symmetric
  integer interval [-7, 7]; -8 is never produced for |w| <= max|w|), stored
  as the unsigned nibble q = c + 8 (offset binary).  No zeros are stored; the
  dequant below then runs with z = 8, which gives w = c * s.
* Dequant: w = round16((q - z) * s) with the product formed exactly in fp32
  (a 5-bit integer times an 11-bit significand) and rounded once to the output
  type (fp16 or bf16, nearest-even).  Scales and zeros are gathered through
  ``g_idx`` (group of column k = g_idx[k]; default k // G).
"""

import numpy as np

from .fp import round_to

SYM_ZERO = 8   # implicit zero of a symmetric code (offset-binary storage)


def default_g_idx(K, group_size):
    return (np.arange(K, dtype=np.int64) // group_size).astype(np.int32)


def quantize_rtn_int4(W, group_size=128, g_idx=None, sym=False):
    """RTN-quantize W [N, K] fp32 into codes, fp16 scales and zeros.

    Returns (q uint8 [N, K], scales fp16 [K/G, N], zeros uint8 [K/G, N]);
    ``sym=True`` returns zeros = None (codes are offset by SYM_ZERO).
    A group is the set {k : g_idx[k] == g} (default: G consecutive columns).
    """
    W = np.asarray(W, dtype=np.float32)
    N, K = W.shape
    G = int(group_size)
    assert K % G == 0
    ng = K // G
    gi = default_g_idx(K, G) if g_idx is None else np.asarray(g_idx, dtype=np.int64)
    q = np.zeros((N, K), dtype=np.uint8)
    scales = np.zeros((ng, N), dtype=np.float16)
    zeros = None if sym else np.zeros((ng, N), dtype=np.uint8)
    fifteen, seven = np.float32(15.0), np.float32(7.0)
    for g in range(ng):
        cols = np.nonzero(gi == g)[0]
        Wg = W[:, cols]                                   # [N, |g|] fp32
        if sym:
            s32 = np.abs(Wg).max(axis=1) / seven          # fp32 divide
        else:
            mn = Wg.min(axis=1)
            mx = Wg.max(axis=1)
            s32 = (mx - mn) / fifteen                     # fp32 subtract, fp32 divide
        s16 = s32.astype(np.float16)                      # RNE to fp16
        s16 = np.where(s16 == 0, np.float16(1.0), s16)    # degenerate group
        sf = s16.astype(np.float32)
        if sym:
            c = np.clip(np.rint(Wg / sf[:, None]), -8, 7)  # half-even
            q[:, cols] = (c + SYM_ZERO).astype(np.uint8)
        else:
            z = np.clip(np.rint(-mn / sf), 0, 15)         # fp32 divide, half-even
            qg = np.clip(np.rint(Wg / sf[:, None]) + z[:, None], 0, 15)
            q[:, cols] = qg.astype(np.uint8)
            zeros[g] = z.astype(np.uint8)
        scales[g] = s16
    return q, scales, zeros


def pack_qweight(q):
    """Codes [N, K] (0..15) -> int32 [K/8, N], 8 codes per word along K."""
    q = np.asarray(q, dtype=np.uint32)
    N, K = q.shape
    assert K % 8 == 0
    qt = q.T.reshape(K // 8, 8, N)
    w = np.zeros((K // 8, N), dtype=np.uint32)
    for j in range(8):
        w |= qt[:, j, :] << np.uint32(4 * j)
    return w.view(np.int32)


def unpack_qweight(qweight):
    """int32 [K/8, N] -> codes uint8 [N, K] (logical shifts on uint32)."""
    w = np.asarray(qweight).view(np.uint32)
    K8, N = w.shape
    out = np.zeros((K8, 8, N), dtype=np.uint8)
    for j in range(8):
        out[:, j, :] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(K8 * 8, N).T.copy()


def pack_qzeros(z):
    """Zeros [K/G, N] -> int32 [K/G, N/8], 8 zeros per word along N."""
    z = np.asarray(z, dtype=np.uint32)
    ng, N = z.shape
    assert N % 8 == 0
    zr = z.reshape(ng, N // 8, 8)
    w = np.zeros((ng, N // 8), dtype=np.uint32)
    for j in range(8):
        w |= zr[:, :, j] << np.uint32(4 * j)
    return w.view(np.int32)


def unpack_qzeros(qzeros):
    """int32 [K/G, N/8] -> zeros uint8 [K/G, N]."""
    w = np.asarray(qzeros).view(np.uint32)
    ng, N8 = w.shape
    out = np.zeros((ng, N8, 8), dtype=np.uint8)
    for j in range(8):
        out[:, :, j] = (w >> np.uint32(4 * j)) & np.uint32(0xF)
    return out.reshape(ng, N8 * 8)


def dequant_int4(qweight, scales, qzeros, g_idx=None, group_size=128, dtype="f16"):
    """Dequantize canonical GPTQ-style tensors to W_deq [N, K] as uint16 bits.

    w[n, k] = round_dtype(fp32(q[n,k] - z[g,n]) * fp32(s[g,n])), g = g_idx[k];
    ``qzeros=None`` is a symmetric weight (z = SYM_ZERO everywhere).
    """
    q = unpack_qweight(qweight)
    z = None if qzeros is None else unpack_qzeros(qzeros)[:, :q.shape[0]]
    return dequant_codes(q, scales, z, g_idx, group_size, dtype)


def dequant_codes(q, scales, zeros, g_idx=None, group_size=128, dtype="f16"):
    """Same definition on unpacked codes q [N, K], scales [K/G, N], zeros [K/G, N]
    (or None: symmetric, z = SYM_ZERO)."""
    q = np.asarray(q, dtype=np.uint8)
    N, K = q.shape
    s = np.asarray(scales, dtype=np.float16)
    z = (np.full(s.shape, SYM_ZERO, dtype=np.uint8) if zeros is None
         else np.asarray(zeros, dtype=np.uint8))
    gi = default_g_idx(K, group_size) if g_idx is None else np.asarray(g_idx, dtype=np.int64)
    zk = z[gi, :].T.astype(np.float32)                    # [N, K]
    sk = s[gi, :].T.astype(np.float32)                    # [N, K]
    prod = (q.astype(np.float32) - zk) * sk               # exact in fp32
    return round_to(prod, dtype)
