"""Helpers shared by the GPU parity tests (inputs from synth, expectations
from the oracle only)."""

import sys

import numpy as np
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import int4, nf4, gemm, fp

DEV = "cuda"
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def bits_to_tensor(bits, dtype):
    t = torch.from_numpy(np.ascontiguousarray(bits).view(np.int16).copy())
    return t.view(TDT[dtype]).to(DEV)


def tensor_bits(t):
    return t.detach().contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def tensor_f64(t, dtype):
    return fp.bits_to_f64(tensor_bits(t), dtype)


def int4_inputs(tag, N, K, act_order=False, awq=False):
    """fp32 W [N, K] (AWQ-folded if asked), optional g_idx, and AWQ scales."""
    W = synth.weights(tag + "/W", N, K)
    s = None
    if awq:
        s = synth.awq_scales(tag + "/s", K)
        W = (W * s[None, :]).astype(np.float32)
    gi = synth.act_order_gidx(tag + "/g", K, 128) if act_order else None
    return W, gi, s


def gpu_int4_pack(W, gi):
    """Product path: device quantizer + device repack."""
    Wd = torch.from_numpy(W).to(DEV)
    gid = torch.from_numpy(gi).to(DEV) if gi is not None else None
    qw, sc, qz = w4.w4a16_quantize_rtn(Wd, 128, g_idx=gid)
    packed = w4.w4a16_repack(qw, sc, qz, gid)
    return (qw, sc, qz), packed


def oracle_int4_rows(W, gi, rows, dtype):
    """Oracle dequantized weights [len(rows), K] for a subset of output rows,
    in the original input-column order (rows are quantized independently)."""
    q, s, z = int4.quantize_rtn_int4(W[rows], 128, gi)
    wd = int4.dequant_codes(q, s, z, gi, 128, dtype)
    return wd


def compare_gemm(y_gpu, x_bits, wd_bits, dtype, cols=None):
    """Relative error of GPU outputs (optionally a column subset) vs fp64 oracle."""
    y_ref = gemm.gemm_ref_bits(x_bits, wd_bits, dtype)
    y = tensor_f64(y_gpu, dtype)
    if cols is not None:
        y = y[:, cols]
    return gemm.rel_err(y, y_ref)
