"""fp64 reference product and the relative-error score (test infrastructure only).

The fused kernel reaches, up to the order of its fp32 accumulation, the plain
product of the activations with the dequantized weights: y = x * dequant(Wq)^T
(the fused dequantize-and-multiply of [P5] "关键数据解读" item 1).  The oracle is
that definition: both operands widened exactly to fp64, one matmul.

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


def rel_err(y, y_ref):
    y = np.asarray(y, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    den = np.max(np.abs(y_ref)) if y_ref.size else 0.0
    num = np.max(np.abs(y - y_ref)) if y_ref.size else 0.0
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
