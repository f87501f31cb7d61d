"""fp64 reference product and the relative-error score (test infrastructure only).

The fused kernel reaches, up to the order of its fp32 accumulation, the plain
product of the activations with the dequantized weights: y = x * dequant(Wq)^T
(the fused dequantize-and-multiply of [P5] "关键数据解读" item 1).  The oracle is
that definition: both operands widened exactly to fp64, one matmul.

AWQ input scales ([P3] §4.1: a salient input channel's weights are scaled up
by s_k before quantization and its activations divided by s_k): with the
division applied by the GEMM itself the product is
y = sum_k (x[:, k] / s_k) * w[:, k]; the oracle evaluates it in fp64, with
no intermediate rounding of x / s (the kernel's rounding of x / s to its
16-bit operand type is part of what the score bounds).

Score (the pass bar): max|y - y_ref| / max|y_ref| over all M x N outputs of a
call, with y widened exactly to fp64; the bar is 5e-3.
"""

import numpy as np

from .fp import bits_to_f64

TOL = 5e-3


def gemm_ref_fp64(x64, w64):
    """y_ref = x64 @ w64^T in fp64.  x64 [M, K], w64 [N, K] (exact fp64 values)."""
    x64 = np.asarray(x64, dtype=np.float64)
    w64 = np.asarray(w64, dtype=np.float64)
    return x64 @ w64.T


def gemm_ref_bits(x_bits, w_bits, dtype, perm=None):
    """Reference product from 16-bit operand bit patterns of ``dtype``.

    ``perm`` (optional) gathers activation columns: x_p[:, j] = x[:, perm[j]],
    for weights stored in permuted column order.
    """
    x = bits_to_f64(x_bits, dtype)
    if perm is not None:
        x = x[:, np.asarray(perm)]
    return gemm_ref_fp64(x, bits_to_f64(w_bits, dtype))


def gemm_ref_xscale_bits(x_bits, s_bits, w_bits, dtype, perm=None):
    """y_ref = (x / s) @ w^T in fp64, s [K] the per-input-channel AWQ scales
    (16-bit bits of ``dtype``, indexed by ORIGINAL input channel); ``perm``
    as in gemm_ref_bits (the division happens before the gather)."""
    x = bits_to_f64(x_bits, dtype)
    s = bits_to_f64(np.asarray(s_bits).reshape(1, -1), dtype)
    xs = x / s
    if perm is not None:
        xs = xs[:, np.asarray(perm)]
    return gemm_ref_fp64(xs, bits_to_f64(w_bits, dtype))


def rel_err(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    num = np.max(np.abs(y - y_ref)) if y_ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
