"""Parity of the large-M (prefill) INT4 kernel with the oracle.

w4a16_gemm switches to the LDS-staged kernel for M >= 32 rows, 5 on layers
of 100 Mi weights and 16 or 24 on layers of 24 Mi weights (32-, 64-, 128-,
192- or 256-row workgroup tiles, K split over workgroups with an ordered reduction of
fp32 partials when that fills the GPU better); these cases cover several
workgroup tiles, ragged row blocks, a panel count that is not a multiple of 4
(N = 320 -> 5 panels), act-order, split K, bf16 with outlier channels, and
exact one-hot probes through the kernel.
"""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle.gemm import TOL
from gpu_util import (say, bits_to_tensor, tensor_bits, int4_inputs, gpu_int4_pack,
                      oracle_int4_rows, compare_gemm)

pytestmark = pytest.mark.gpu


def _gemm(tag, M, N, K, dtype, act=False, outliers=False):
    W, gi, _ = int4_inputs(tag, N, K, act_order=act)
    x32 = synth.activations(tag + "/x", M, K)
    if outliers:
        x32 = synth.with_outliers(x32, synth.outlier_channels(tag + "/outl", K))
    xb = synth.to_bits(x32, dtype)
    _, packed = gpu_int4_pack(W, gi)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    return y, xb, W, gi, packed


@pytest.mark.parametrize("M", [256, 257, 600])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_ragged(M, dtype):
    N, K = 320, 640
    say("prefill", M, dtype)
    y, xb, W, gi, _ = _gemm("gpu/pf/%d" % M, M, N, K, dtype)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    assert compare_gemm(y, xb, wd, dtype) <= TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_act_order(dtype):
    M, N, K = 300, 512, 1024
    say("prefill act", dtype)
    y, xb, W, gi, _ = _gemm("gpu/pf/act", M, N, K, dtype, act=True)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    assert compare_gemm(y, xb, wd, dtype) <= TOL


def test_prefill_bf16_outlier_channels_sampled_columns():
    # bf16 activations with 1 % of input channels x20, several K tiles and
    # row blocks; the oracle checks every 5th output column
    M, N, K = 1024, 1280, 2560
    say("prefill outliers")
    y, xb, W, gi, _ = _gemm("gpu/pf/outl", M, N, K, "bf16", outliers=True)
    cols = np.arange(0, N, 5)
    wd = oracle_int4_rows(W, gi, cols, "bf16")
    assert compare_gemm(y, xb, wd, "bf16", cols=cols) <= TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_prefill_onehot_exact(dtype):
    # 256 one-hot rows: every output equals one dequantized weight bit for bit
    N, K = 320, 512
    W, gi, _ = int4_inputs("gpu/pf/onehot", N, K, act_order=True)
    _, packed = gpu_int4_pack(W, gi)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    M = 256
    ks = (np.arange(M) * 37) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, dtype), dtype), packed))
    assert np.array_equal(y, wd[:, ks].T)


def test_prefill_deterministic():
    M, N, K = 512, 256, 1024
    W, gi, _ = int4_inputs("gpu/pf/det", N, K)
    _, packed = gpu_int4_pack(W, gi)
    x = bits_to_tensor(synth.to_bf16_bits(synth.activations("gpu/pf/det/x", M, K)), "bf16")
    y1 = tensor_bits(w4.w4a16_gemm(x, packed))
    y2 = tensor_bits(w4.w4a16_gemm(x, packed))
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("M", [64, 65, 100, 128, 129, 200])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_mid_m_split_k(M, dtype):
    # small row counts: 64/128-row tiles and, for so few workgroups, K split
    # over workgroups (partials through the workspace)
    N, K = 320, 2560
    say("mid M", M, dtype, "workspace", w4.w4a16_workspace_bytes(M, N, K))
    y, xb, W, gi, _ = _gemm("gpu/pf/mid/%d" % M, M, N, K, dtype)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    assert compare_gemm(y, xb, wd, dtype) <= TOL


def test_mid_m_act_order_and_determinism():
    M, N, K = 96, 256, 3072
    W, gi, _ = int4_inputs("gpu/pf/midact", N, K, act_order=True)
    _, packed = gpu_int4_pack(W, gi)
    xb = synth.to_f16_bits(synth.activations("gpu/pf/midact/x", M, K))
    y1 = w4.w4a16_gemm(bits_to_tensor(xb, "f16"), packed)
    y2 = w4.w4a16_gemm(bits_to_tensor(xb, "f16"), packed)
    assert np.array_equal(tensor_bits(y1), tensor_bits(y2))
    wd = oracle_int4_rows(W, gi, np.arange(N), "f16")
    assert compare_gemm(y1, xb, wd, "f16") <= TOL


def test_mid_m_onehot_exact_through_split_k():
    # one-hot rows through the split-K path: each output is one weight plus
    # exact zeros from the other splits
    N, K = 256, 4096
    W, gi, _ = int4_inputs("gpu/pf/midonehot", N, K)
    _, packed = gpu_int4_pack(W, gi)
    wd = oracle_int4_rows(W, gi, np.arange(N), "bf16")
    M = 64
    ks = (np.arange(M) * 61) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    assert w4.w4a16_workspace_bytes(M, N, K) > 0          # this shape splits K
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, "bf16"), "bf16"), packed))
    assert np.array_equal(y, wd[:, ks].T)


def test_big_layer_m16_uses_large_m_kernel_sampled_columns():
    # 16 rows on a 100 Mi-weight layer take the large-M kernel with split K;
    # the oracle checks every 97th output column
    M, N, K = 16, 20480, 5120
    say("big layer M=16")
    y, xb, W, gi, _ = _gemm("gpu/pf/big16", M, N, K, "bf16")
    cols = np.arange(0, N, 97)
    wd = oracle_int4_rows(W, gi, cols, "bf16")
    assert compare_gemm(y, xb, wd, "bf16", cols=cols) <= TOL


@pytest.mark.parametrize("M,N,K,dtype", [(5, 20480, 5120, "f16"), (4, 20480, 5120, "bf16"),
                                         (32, 11008, 4096, "bf16"), (31, 11008, 4096, "f16"),
                                         (17, 4096, 11008, "bf16"), (16, 4096, 11008, "f16")])
def test_kernel_crossover_rows_act_order_sampled_columns(M, N, K, dtype):
    # the fewest rows that take the large-M kernel (32-row workgroup tiles)
    # on a 100 Mi-weight layer (5) and on 43 Mi-weight layers (32 with 11008
    # columns, 17 with 4096), and one row fewer (the decode kernel),
    # act-order; every 61st output column
    say("crossover", M, N, K, dtype)
    y, xb, W, gi, _ = _gemm("gpu/pf/cross/%d" % M, M, N, K, dtype, act=True)
    cols = np.arange(3, N, 61)
    wd = oracle_int4_rows(W, gi, cols, dtype)
    assert compare_gemm(y, xb, wd, dtype, cols=cols) <= TOL
