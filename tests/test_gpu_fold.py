"""GPU parity of the kernel paths that apply the scale and zero after the K sum
(the decode kernel's packed modes, M <= 4, and its FULLT mode with one row
tile, M <= 16 with G >= 128; the large-M kernel's 32-row tiles, M <= 32):
one-hot rows exact for every group size and code form, and
activations with large outlier channels within the tolerance (the o + q
operands put o x in every partial sum, which the fold subtracts again)."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import intb, gemm
from gpu_util import DEV, say, bits_to_tensor, tensor_bits, compare_gemm

pytestmark = pytest.mark.gpu
TOL = gemm.TOL


def _pack(W, bits, G, gi, sym):
    Wd = torch.from_numpy(W).to(DEV)
    gid = torch.from_numpy(gi).to(DEV) if gi is not None else None
    qw, sc, qz = w4.w4a16_quantize_rtn(Wd, G, g_idx=gid, sym=sym, bits=bits)
    return w4.w4a16_repack(qw, sc, qz, gid, G, bits=bits)


def _wd(W, bits, G, gi, sym, dtype):
    K = W.shape[1]
    g = K if G == -1 else G
    q, s, z = intb.quantize_rtn(W, bits, g, gi, sym)
    return intb.dequant_codes(q, s, z, bits, gi, g, dtype)


# (bits, G, sym, act): the packed fold selects the meta unit of each lane's
# MFMA step, so every group size goes through it
CASES = [(4, 128, False, True), (4, 64, True, False), (4, 32, False, True), (4, -1, True, False),
         (3, 128, False, False), (8, 64, False, True)]


@pytest.mark.parametrize("bits,G,sym,act", CASES)
@pytest.mark.parametrize("M", [1, 3, 12, 32])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fold_onehot_exact(bits, G, sym, act, M, dtype):
    N, K = 160, 1024
    say("fold onehot", bits, G, sym, act, M, dtype)
    tag = "gpu/fold/oh/%d/%d" % (bits, G)
    W = synth.weights(tag + "/W", N, K)
    gi = synth.act_order_gidx(tag + "/g", K, G) if act and G != -1 else None
    packed = _pack(W, bits, G, gi, sym)
    wd = _wd(W, bits, G, gi, sym, dtype)
    ks = (np.arange(M) * 131 + 17) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, dtype), dtype), packed))
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wd[:, k]), (r, k)


@pytest.mark.parametrize("bits,G,sym,act", CASES)
@pytest.mark.parametrize("M", [2, 4, 12, 32])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_fold_outlier_channels(bits, G, sym, act, M, dtype):
    # 1 % of the input channels x20 and four channels scaled further (x 2^8 in
    # fp16, which keeps them finite, x 2^40 in bf16)
    N, K = 224, 2048
    say("fold outliers", bits, G, sym, act, M, dtype)
    tag = "gpu/fold/out/%d/%d/%d" % (bits, G, M)
    W = synth.weights(tag + "/W", N, K)
    gi = synth.act_order_gidx(tag + "/g", K, G) if act and G != -1 else None
    packed = _pack(W, bits, G, gi, sym)
    x32 = synth.with_outliers(synth.activations(tag + "/x", M, K),
                              synth.outlier_channels(tag + "/oc", K))
    big = np.array([5, 700, 1500, 2047])
    x32[:, big] *= 2.0 ** (8 if dtype == "f16" else 40)
    xb = synth.to_bits(x32, dtype)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    err = compare_gemm(y, xb, _wd(W, bits, G, gi, sym, dtype), dtype)
    say("  rel err", err)
    assert err <= TOL


# wide layers (N >= 16384): the packed decode runs 2 column tiles per wave for
# 3 or 4 rows (M = 1: the one-tile kernel); N = 16416 leaves a partly filled
# last panel
WIDE = [(4, 128, False, True), (4, 32, True, False), (3, 64, False, False), (8, 128, True, False)]


@pytest.mark.parametrize("bits,G,sym,act", WIDE)
@pytest.mark.parametrize("M", [1, 3, 4])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_wide_layer_sampled_columns(bits, G, sym, act, M, dtype):
    N, K = 16416, 1024
    say("fold wide", bits, G, sym, act, M, dtype)
    tag = "gpu/fold/wide/%d/%d" % (bits, G)
    W = synth.weights(tag + "/W", N, K)
    gi = synth.act_order_gidx(tag + "/g", K, G) if act else None
    packed = _pack(W, bits, G, gi, sym)
    xb = synth.to_bits(synth.activations(tag + "/x/%d" % M, M, K), dtype)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    cols = np.unique(np.concatenate([np.arange(0, N, 97), np.arange(N - 40, N)]))
    K_ = W.shape[1]
    g = K_ if G == -1 else G
    q, s, z = intb.quantize_rtn(W[cols], bits, g, gi, sym)
    wd = intb.dequant_codes(q, s, z, bits, gi, g, dtype)
    assert compare_gemm(y, xb, wd, dtype, cols=cols) <= TOL


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_wide_layer_onehot_exact(dtype):
    N, K, G = 16416, 512, 128
    say("fold wide onehot", dtype)
    W = synth.weights("gpu/fold/wide/oh", N, K)
    gi = synth.act_order_gidx("gpu/fold/wide/oh/g", K, G)
    packed = _pack(W, 4, G, gi, False)
    ks = np.array([3, 200, 511, 77])
    x = np.zeros((4, K), dtype=np.float32)
    x[np.arange(4), ks] = 1.0
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, dtype), dtype), packed))
    cols = np.unique(np.concatenate([np.arange(0, N, 61), np.arange(N - 40, N)]))
    q, s, z = intb.quantize_rtn(W[cols], 4, G, gi, False)
    wd = intb.dequant_codes(q, s, z, 4, gi, G, dtype)
    for r, k in enumerate(ks):
        assert np.array_equal(y[r][cols], wd[:, k]), (r, k)
