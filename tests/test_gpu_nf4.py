"""GPU parity of the NF4 path: on-device quantizer and dequant bit-exact vs the
oracle; fused GEMM within the 5e-3 relative bar."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import nf4, gemm
from gpu_util import DEV, say, bits_to_tensor, tensor_bits, compare_gemm

pytestmark = pytest.mark.gpu
TOL = gemm.TOL


def _pack(W):
    return w4.nf4_quantize(torch.from_numpy(W).to(DEV), 64)


@pytest.mark.parametrize("N,K", [(64, 512), (48, 192), (512, 1024)])
def test_nf4_quantizer_bit_exact(N, K):
    say("nf4 quant", N, K)
    W = synth.weights("gpu/nf4q/%d/%d" % (N, K), N, K)
    W[1, :64] = 0.0                                   # an all-zero block
    p = _pack(W)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    assert np.array_equal(p["qweight"].cpu().numpy(), nf4.pack_nf4(codes))
    assert np.array_equal(p["absmax_q"].cpu().numpy(), aq)
    assert np.array_equal(p["absmax_scale"].cpu().numpy().view(np.uint32), sc.view(np.uint32))


@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nf4_dequant_bit_exact(dtype):
    N, K = 96, 1024
    say("nf4 dequant", dtype)
    W = synth.weights("gpu/nf4d", N, K)
    p = _pack(W)
    got = tensor_bits(w4.nf4_dequant(p, torch.bfloat16 if dtype == "bf16" else torch.float16))
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    want = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, dtype)
    assert np.array_equal(got, want)


@pytest.mark.parametrize("M", [1, 2, 16, 17, 32, 33, 64, 70])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nf4_gemm(M, dtype):
    N, K = 208, 1088                          # ragged: N % 64 != 0, K % 128 == 64
    say("nf4 gemm", M, dtype)
    W = synth.weights("gpu/nf4g/W", N, K)
    x32 = synth.activations("gpu/nf4g/x/%d" % M, M, K)
    xb = synth.to_bits(x32, dtype)
    p = _pack(W)
    y = w4.nf4_gemm(bits_to_tensor(xb, dtype), p)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, dtype)
    assert compare_gemm(y, xb, wd, dtype) <= TOL


def test_nf4_gemm_onehot_exact():
    N, K = 64, 512
    W = synth.weights("gpu/nf4/onehot", N, K)
    p = _pack(W)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, "bf16")
    ks = [0, 5, 63, 64, 200, 511]
    x = np.zeros((len(ks), K), dtype=np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = tensor_bits(w4.nf4_gemm(bits_to_tensor(synth.to_bf16_bits(x), "bf16"), p))
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wd[:, k]), k


@pytest.mark.parametrize("M", [1, 3, 4, 5, 16, 40])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nf4_gemm_k_multiple_of_1024(M, dtype):
    # K % 1024 == 0: the kernel reads the 16 absmax codes of 8 K tiles at once
    N, K = 144, 3072
    say("nf4 gemm k1024", M, dtype)
    W = synth.weights("gpu/nf4k/W", N, K)
    xb = synth.to_bits(synth.activations("gpu/nf4k/x/%d" % M, M, K), dtype)
    p = _pack(W)
    y = w4.nf4_gemm(bits_to_tensor(xb, dtype), p)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, dtype)
    assert compare_gemm(y, xb, wd, dtype) <= TOL


def test_nf4_gemm_onehot_exact_k1024():
    N, K = 32, 1024
    W = synth.weights("gpu/nf4/onehot1024", N, K)
    p = _pack(W)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, "f16")
    ks = [0, 127, 128, 500, 1023]
    x = np.zeros((len(ks), K), dtype=np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = tensor_bits(w4.nf4_gemm(bits_to_tensor(synth.to_f16_bits(x), "f16"), p))
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wd[:, k]), k


@pytest.mark.parametrize("M", [12, 32, 64, 96, 300])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nf4_gemm_large_m(M, dtype):
    # the large-M kernel (K % 128 == 0): 32 x 32 MFMA tiles with the NF4 codes
    # read from the canonical layout, split K where the grid is small
    N, K = 160, 2048
    say("nf4 large M", M, dtype, "workspace", w4.nf4_workspace_bytes(M, N, K))
    W = synth.weights("gpu/nf4L/W", N, K)
    xb = synth.to_bits(synth.activations("gpu/nf4L/x/%d" % M, M, K), dtype)
    p = _pack(W)
    y = w4.nf4_gemm(bits_to_tensor(xb, dtype), p)
    # without a workspace: the large-M kernel does not split K
    y0 = w4.nf4_gemm(bits_to_tensor(xb, dtype), p, use_workspace=False)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, dtype)
    assert compare_gemm(y, xb, wd, dtype) <= TOL
    assert compare_gemm(y0, xb, wd, dtype) <= TOL


def test_nf4_large_m_onehot_exact():
    N, K = 96, 1024
    W = synth.weights("gpu/nf4L/onehot", N, K)
    p = _pack(W)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, "bf16")
    M = 64
    ks = (np.arange(M) * 37 + 5) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = tensor_bits(w4.nf4_gemm(bits_to_tensor(synth.to_bf16_bits(x), "bf16"), p))
    assert np.array_equal(y, wd[:, ks].T)


@pytest.mark.parametrize("N,M", [(16416, 3), (16416, 4), (16400, 4)])
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_nf4_wide_layer_sampled_columns(N, M, dtype):
    # wide layers through the NF4 packed decode (the integer formats run 2
    # column tiles per wave from N = 16384 on; NF4 keeps one, its dequant
    # being the bound); every 53rd output column and the last 40
    K = 1024
    say("nf4 wide", N, M, dtype)
    W = synth.weights("gpu/nf4W/W", N, K)
    xb = synth.to_bits(synth.activations("gpu/nf4W/x/%d" % M, M, K), dtype)
    p = _pack(W)
    y = w4.nf4_gemm(bits_to_tensor(xb, dtype), p)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([np.arange(0, N, 53), np.arange(N - 40, N)]))
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, dtype)[cols]
    assert compare_gemm(y, xb, wd, dtype, cols=cols) <= TOL


@pytest.mark.parametrize("M", [12, 20])
def test_nf4_full_rows_onehot_exact_ragged_k(M):
    # the decode kernel's whole-line loads and LDS transpose with a half last
    # K tile (K % 128 == 64): every output is one dequantized weight
    N, K = 80, 1088
    say("nf4 full-row onehot", M)
    W = synth.weights("gpu/nf4/fullrow", N, K)
    p = _pack(W)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, "bf16")
    ks = (np.arange(M) * 91 + 1087) % K          # includes k = 1087, in the half tile
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = tensor_bits(w4.nf4_gemm(bits_to_tensor(synth.to_bf16_bits(x), "bf16"), p))
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wd[:, k]), (r, k)
