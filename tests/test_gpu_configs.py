"""GPU parity at the full sizes of the benchmark workloads, in the launch
configuration bench.py times (weights quantized and repacked on the device),
against the oracle evaluated on the same inputs (its own quantizer, dequant
and fp64 product, row chunk by row chunk), within
max|y - y_ref| / max|y_ref| <= 5e-3 with both maxima over the compared
outputs:

* Llama-2-7B-shaped decode, GPTQ act-order int4 G=128, fp16, M in {1, 4, 16}:
  the whole output;
* Qwen2.5-32B-shaped decode layers in AWQ layout (s ~ U[0.5, 2] folded into
  W, x divided by s), int4 G=128, fp16, M in {1, 16, 64}, and the same layers
  with the raw activations and s passed to w4a16_gemm_xscale: the whole
  output;
* the same four layers in prefill, bf16 with 1 % outlier channels x20,
  M in {2048, 8192}: every 8th output column of every row, and the whole
  output of 5120 x 5120 at M = 2048;
* NF4 28672 x 8192, bf16, M in {1, 15, 32, 33}: the whole output.
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
CHUNK = 8192                                                   # weight rows per oracle chunk


def _int4_ref(Wf, gi, dtype, xs, cols=None, x_scale_bits=None):
    """Oracle outputs y_ref[m][:, cols] for each activation set of xs (bits),
    dequantizing the weight rows of `cols` chunk by chunk."""
    N = Wf.shape[0]
    cols = np.arange(N) if cols is None else cols
    outs = [np.empty((x.shape[0], cols.size)) for x in xs]
    for c0 in range(0, cols.size, CHUNK):
        rows = cols[c0:c0 + CHUNK]
        q, s, z = int4.quantize_rtn_int4(Wf[rows], G, gi)
        wd = int4.dequant_codes(q, s, z, gi, G, dtype)
        for o, x in zip(outs, xs):
            o[:, c0:c0 + rows.size] = (gemm.gemm_ref_bits(x, wd, dtype) if x_scale_bits is None
                                       else gemm.gemm_ref_xscale_bits(x, x_scale_bits, wd, dtype))
    return outs


@pytest.mark.parametrize("K,N", LLAMA)
def test_llama2_7b_decode_actorder(K, N):
    say("config llama decode", K, N)
    W = synth.weights("C2/W/%dx%d" % (K, N), N, K)
    gi = synth.act_order_gidx("C2/gidx/%dx%d" % (K, N), K, G)
    gid = torch.from_numpy(gi).to(DEV)
    qw, sc, qz = w4.w4a16_quantize_rtn(torch.from_numpy(W).to(DEV), G, g_idx=gid)
    packed = w4.w4a16_repack(qw, sc, qz, gid)
    Ms = (1, 4, 16)
    xs = [synth.to_f16_bits(synth.activations("C2/x/%dx%d" % (M, K), M, K)) for M in Ms]
    refs = _int4_ref(W, gi, "f16", xs)
    for M, xb, y_ref in zip(Ms, xs, refs):
        y = w4.w4a16_gemm(bits_to_tensor(xb, "f16"), packed)
        err = gemm.rel_err(tensor_f64(y, "f16"), y_ref)
        say("  M", M, w4.w4a16_gemm_plan(M, N, K, perm=True), "rel err (whole output)", err)
        assert err <= TOL, (M, err)


@pytest.mark.parametrize("K,N", QWEN)
def test_qwen2_5_32b_decode_awq_layout(K, N):
    say("config qwen decode awq", K, N)
    W = synth.weights("C3/W/%dx%d" % (K, N), N, K)
    s32 = synth.awq_scales("C3/s/%d" % K, K)
    sb = synth.to_f16_bits(s32[None, :])[0]
    sf = fp.bits_to_f64(sb, "f16")
    Wf = (W.astype(np.float64) * sf[None, :]).astype(np.float32)      # W' = W s
    del W
    qw, sc, qz = w4.w4a16_quantize_rtn(torch.from_numpy(Wf).to(DEV), G)
    packed = w4.w4a16_repack(qw, sc, qz)
    del qw, sc, qz
    Ms = (1, 16, 64)
    xbs = [synth.to_f16_bits(synth.activations("C3/x/%dx%d" % (M, K), M, K)) for M in Ms]
    # the AWQ layout: x divided by s before the call ...
    xdbs = [synth.to_f16_bits((fp.bits_to_f64(xb, "f16") / sf[None, :]).astype(np.float32))
            for xb in xbs]
    refs = _int4_ref(Wf, None, "f16", xdbs)
    # ... or the raw x with s, divided by the GEMM itself
    refs2 = _int4_ref(Wf, None, "f16", xbs, x_scale_bits=sb)
    del Wf
    for M, xb, xdb, y_ref, y_ref2 in zip(Ms, xbs, xdbs, refs, refs2):
        y = w4.w4a16_gemm(bits_to_tensor(xdb, "f16"), packed)
        err = gemm.rel_err(tensor_f64(y, "f16"), y_ref)
        y2 = w4.w4a16_gemm_xscale(bits_to_tensor(xb, "f16"), bits_to_tensor(sb, "f16"), packed)
        err2 = gemm.rel_err(tensor_f64(y2, "f16"), y_ref2)
        say("  M", M, w4.w4a16_gemm_plan(M, N, K), "rel err (whole output)", err,
            "with x_scale", err2)
        assert err <= TOL and err2 <= TOL, (M, err, err2)


@pytest.mark.parametrize("K,N", QWEN)
def test_qwen2_5_32b_prefill_outliers(K, N):
    say("config qwen prefill", K, N)
    W = synth.weights("C4/W/%dx%d" % (K, N), N, K)
    qw, sc, qz = w4.w4a16_quantize_rtn(torch.from_numpy(W).to(DEV), G)
    packed = w4.w4a16_repack(qw, sc, qz)
    del qw, sc, qz
    every8 = np.arange(0, N, 8)
    for M in (2048, 8192):
        x32 = synth.activations("C4/x/%dx%d" % (M, K), M, K)
        x32 = synth.with_outliers(x32, synth.outlier_channels("C4/outl/%d" % K, K))
        xb = synth.to_bf16_bits(x32)
        del x32
        y = w4.w4a16_gemm(bits_to_tensor(xb, "bf16"), packed)
        torch.cuda.synchronize()
        whole = (K, N) == (5120, 5120) and M == 2048
        cols = np.arange(N) if whole else every8
        (y_ref,) = _int4_ref(W, None, "bf16", [xb], cols=cols)
        err = gemm.rel_err(tensor_f64(y, "bf16")[:, cols], y_ref)
        say("  M", M, w4.w4a16_gemm_plan(M, N, K, dtype=torch.bfloat16),
            "rel err (%s)" % ("whole output" if whole else "every 8th column"), err)
        assert err <= TOL, (M, err)
        del y, xb, y_ref
        torch.cuda.empty_cache()


def test_nf4_28672x8192():
    N, K = 28672, 8192
    say("config nf4")
    W = synth.weights("C5/W", N, K)
    t = w4.nf4_quantize(torch.from_numpy(W).to(DEV))
    L = nf4.nf4_codebook()
    Ms = (1, 15, 32, 33)     # up to 32: the decode kernel, 33: the large-M kernel
    xs = [synth.to_bf16_bits(synth.activations("C5/x/%d" % M, M, K)) for M in Ms]
    refs = [np.empty((M, N)) for M in Ms]
    # a double-quant group is 256 blocks of 64 = two rows of K = 8192: chunks
    # of whole row pairs quantize exactly as the whole matrix does
    for r0 in range(0, N, CHUNK):
        codes, absmax = nf4.quantize_nf4(W[r0:r0 + CHUNK], 64, L)
        aq, asc = nf4.double_quant(absmax)
        wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, asc, 64, "bf16", codebook=L)
        for o, xb in zip(refs, xs):
            o[:, r0:r0 + CHUNK] = gemm.gemm_ref_bits(xb, wd, "bf16")
    del W
    for M, xb, y_ref in zip(Ms, xs, refs):
        y = w4.nf4_gemm(bits_to_tensor(xb, "bf16"), t)
        torch.cuda.synchronize()
        err = gemm.rel_err(tensor_f64(y, "bf16"), y_ref)
        say("  M", M, w4.nf4_gemm_plan(M, N, K), "rel err (whole output)", err)
        assert err <= TOL, (M, err)
