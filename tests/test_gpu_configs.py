"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times (weights quantized and repacked on the device):
sampled outputs y[rows][:, cols] against the oracle evaluated for those
rows and columns only, within max|y - y_ref| / max|y_ref| <= 5e-3.

* Llama-2-7B-shaped decode, GPTQ act-order int4 G=128, fp16, M in {1, 4, 16};
* Qwen2.5-32B-shaped decode layers in AWQ layout (s ~ U[0.5, 2] folded into
  W, x divided by s), int4 G=128, fp16, M in {1, 16, 64}; the same layers with
  the raw activations and s passed to w4a16_gemm_xscale;
* the same four layers in prefill, bf16 with 1 % outlier channels x20,
  M in {2048, 8192};
* NF4 28672 x 8192, bf16, M in {1, 15, 16, 32}.
"""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import int4, nf4, gemm, fp
from gpu_util import DEV, say, bits_to_tensor, tensor_f64

pytestmark = pytest.mark.gpu
TOL = gemm.TOL
G = 128
LLAMA = [(4096, 4096), (4096, 11008), (11008, 4096)]          # (K, N)
QWEN = [(5120, 7168), (5120, 5120), (5120, 55296), (27648, 5120)]


def _cols(N, n=48):
    return np.unique(np.concatenate([np.linspace(0, N - 1, n).astype(np.int64), [N - 1]]))


def _rows(M, n=24):
    return np.arange(M) if M <= 64 else np.unique(np.linspace(0, M - 1, n).astype(np.int64))


def _score(y, rows, cols, x_bits, wd_bits, dtype, s_bits=None):
    x = x_bits[rows]
    y_ref = (gemm.gemm_ref_bits(x, wd_bits, dtype) if s_bits is None
             else gemm.gemm_ref_xscale_bits(x, s_bits, wd_bits, dtype))
    got = tensor_f64(y, dtype)[rows][:, cols]
    return gemm.rel_err(got, y_ref)


@pytest.mark.parametrize("K,N", LLAMA)
def test_llama2_7b_decode_actorder(K, N):
    say("config llama decode", K, N)
    W = synth.weights("C2/W/%dx%d" % (K, N), N, K)
    gi = synth.act_order_gidx("C2/gidx/%dx%d" % (K, N), K, G)
    gid = torch.from_numpy(gi).to(DEV)
    qw, sc, qz = w4.w4a16_quantize_rtn(torch.from_numpy(W).to(DEV), G, g_idx=gid)
    packed = w4.w4a16_repack(qw, sc, qz, gid)
    cols = _cols(N)
    q, s, z = int4.quantize_rtn_int4(W[cols], G, gi)
    wd = int4.dequant_codes(q, s, z, gi, G, "f16")
    for M in (1, 4, 16):
        xb = synth.to_f16_bits(synth.activations("C2/x/%dx%d" % (M, K), M, K))
        y = w4.w4a16_gemm(bits_to_tensor(xb, "f16"), packed)
        err = _score(y, _rows(M), cols, xb, wd, "f16")
        say("  M", M, "rel err", err)
        assert err <= TOL, (M, err)


@pytest.mark.parametrize("K,N", QWEN)
def test_qwen2_5_32b_decode_awq_layout(K, N):
    say("config qwen decode awq", K, N)
    W = synth.weights("C3/W/%dx%d" % (K, N), N, K)
    s32 = synth.awq_scales("C3/s/%d" % K, K)
    sb = synth.to_f16_bits(s32[None, :])[0]
    sf = fp.bits_to_f64(sb, "f16")
    Wf = (W.astype(np.float64) * sf[None, :]).astype(np.float32)      # W' = W s
    qw, sc, qz = w4.w4a16_quantize_rtn(torch.from_numpy(Wf).to(DEV), G)
    packed = w4.w4a16_repack(qw, sc, qz)
    del W
    cols = _cols(N)
    q, s, z = int4.quantize_rtn_int4(Wf[cols], G)
    wd = int4.dequant_codes(q, s, z, None, G, "f16")
    for M in (1, 16, 64):
        x32 = synth.activations("C3/x/%dx%d" % (M, K), M, K)
        xb = synth.to_f16_bits(x32)
        # the AWQ layout: x divided by s before the call ...
        xdb = synth.to_f16_bits((fp.bits_to_f64(xb, "f16") / sf[None, :]).astype(np.float32))
        y = w4.w4a16_gemm(bits_to_tensor(xdb, "f16"), packed)
        err = _score(y, _rows(M), cols, xdb, wd, "f16")
        # ... or the raw x with s, divided by the GEMM itself
        y2 = w4.w4a16_gemm_xscale(bits_to_tensor(xb, "f16"), bits_to_tensor(sb, "f16"), packed)
        err2 = _score(y2, _rows(M), cols, xb, wd, "f16", s_bits=sb)
        say("  M", M, "rel err", err, "with x_scale", err2)
        assert err <= TOL and err2 <= TOL, (M, err, err2)


@pytest.mark.parametrize("K,N", QWEN)
def test_qwen2_5_32b_prefill_outliers(K, N):
    say("config qwen prefill", K, N)
    W = synth.weights("C4/W/%dx%d" % (K, N), N, K)
    qw, sc, qz = w4.w4a16_quantize_rtn(torch.from_numpy(W).to(DEV), G)
    packed = w4.w4a16_repack(qw, sc, qz)
    cols = _cols(N, 32)
    q, s, z = int4.quantize_rtn_int4(W[cols], G)
    wd = int4.dequant_codes(q, s, z, None, G, "bf16")
    del W, qw, sc, qz
    for M in (2048, 8192):
        x32 = synth.activations("C4/x/%dx%d" % (M, K), M, K)
        x32 = synth.with_outliers(x32, synth.outlier_channels("C4/outl/%d" % K, K))
        xb = synth.to_bf16_bits(x32)
        del x32
        y = w4.w4a16_gemm(bits_to_tensor(xb, "bf16"), packed)
        torch.cuda.synchronize()
        err = _score(y, _rows(M), cols, xb, wd, "bf16")
        say("  M", M, "rel err", err)
        assert err <= TOL, (M, err)
        del y, xb
        torch.cuda.empty_cache()


def test_nf4_28672x8192():
    N, K = 28672, 8192
    say("config nf4")
    W = synth.weights("C5/W", N, K)
    t = w4.nf4_quantize(torch.from_numpy(W).to(DEV))
    cols = _cols(N)
    L = nf4.nf4_codebook()
    # a double-quant group is 256 blocks of 64 = two rows of K = 8192: the
    # oracle quantizes the aligned row pair of every sampled column
    pairs = np.unique(2 * (cols // 2))
    sub = np.stack([pairs, pairs + 1], axis=1).reshape(-1)
    codes, absmax = nf4.quantize_nf4(W[sub], 64, L)
    aq, asc = nf4.double_quant(absmax)
    wd_sub = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, asc, 64, "bf16", codebook=L)
    wd = wd_sub[2 * np.searchsorted(pairs, 2 * (cols // 2)) + (cols & 1)]
    for M in (1, 15, 32, 33):      # up to 32: the decode kernel, 33: the large-M kernel
        xb = synth.to_bf16_bits(synth.activations("C5/x/%d" % M, M, K))
        y = w4.nf4_gemm(bits_to_tensor(xb, "bf16"), t)
        torch.cuda.synchronize()
        y_ref = gemm.gemm_ref_bits(xb, wd, "bf16")
        err = gemm.rel_err(tensor_f64(y, "bf16")[:, cols], y_ref)
        say("  M", M, "rel err", err)
        assert err <= TOL, (M, err)
