"""GPU parity of 3- and 8-bit integer codes against the oracle (oracle/intb.py,
oracle/repack.py): the device quantizer, repack and dequant bit for bit; the
GEMM within max|y - y_ref| / max|y_ref| <= 5e-3 in every kernel regime, with
act-order and AWQ input scales; one-hot rows exact."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import intb, repack, gemm, fp
from gpu_util import DEV, say, bits_to_tensor, tensor_bits, tensor_f64, compare_gemm

pytestmark = pytest.mark.gpu
TOL = gemm.TOL
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _g(K, G):
    return K if G == -1 else G


def _pack(W, bits, G, gi, sym):
    Wd = torch.from_numpy(W).to(DEV)
    gid = torch.from_numpy(gi).to(DEV) if gi is not None else None
    qw, sc, qz = w4.w4a16_quantize_rtn(Wd, G, g_idx=gid, sym=sym, bits=bits)
    return (qw, sc, qz), w4.w4a16_repack(qw, sc, qz, gid, G, bits=bits)


def _oracle_rows(W, bits, G, gi, sym, rows, dtype):
    K = W.shape[1]
    q, s, z = intb.quantize_rtn(W[rows], bits, _g(K, G), gi, sym)
    return intb.dequant_codes(q, s, z, bits, gi, _g(K, G), dtype)


VARIANTS = [(3, 128, False), (3, 32, True), (3, 64, False), (8, 128, False), (8, 64, True),
            (8, 32, False), (8, -1, True), (3, 256, True)]


@pytest.mark.parametrize("bits,G,sym", VARIANTS)
@pytest.mark.parametrize("act", [False, True])
def test_quantizer_repack_bit_exact(bits, G, sym, act):
    N, K = 224, 1280
    say("bits quantizer+repack", bits, G, sym, act)
    W = synth.weights("gpu/bits/q/%d/%d" % (bits, G), N, K)
    gi = synth.act_order_gidx("gpu/bits/q/g/%d" % G, K, _g(K, G)) if act else None
    (qw, sc, qz), packed = _pack(W, bits, G, gi, sym)
    q, s, z = intb.quantize_rtn(W, bits, _g(K, G), gi, sym)
    assert np.array_equal(qw.cpu().numpy(), intb.pack_qweight(q, bits))
    assert np.array_equal(tensor_bits(sc), s.view(np.uint16))
    if not sym:
        assert np.array_equal(qz.cpu().numpy(), intb.pack_qzeros(z, bits))
    ref = repack.repack_ref_bits(intb.pack_qweight(q, bits), s,
                                 None if sym else intb.pack_qzeros(z, bits), bits, gi, _g(K, G))
    assert np.array_equal(packed["codes"].cpu().numpy(), ref[0])
    assert np.array_equal(tensor_bits(packed["scales"]), ref[1].view(np.uint16))
    if sym:
        assert packed["zeros"] is None
    else:
        assert np.array_equal(packed["zeros"].cpu().numpy().view(np.uint32), ref[2])
    if ref[3] is None:
        assert packed["perm"] is None
    else:
        assert np.array_equal(packed["perm"].cpu().numpy(), ref[3])


@pytest.mark.parametrize("bits,G,sym", VARIANTS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dequant_bit_exact(bits, G, sym, dtype):
    N, K = 160, 2560                     # 2.5 panels of 64 columns; 3-bit zeros need N % 32 == 0
    say("bits dequant", bits, G, sym, dtype)
    W = synth.weights("gpu/bits/deq/%d/%d" % (bits, G), N, K)
    _, packed = _pack(W, bits, G, None, sym)
    got = tensor_bits(w4.w4a16_dequant(packed, TDT[dtype]))
    assert np.array_equal(got, _oracle_rows(W, bits, G, None, sym, np.arange(N), dtype))


# M = 1, 3: packed decode (3 with act-order: gathered on chip); 8: full-row
# decode (act-order: the preparation pass); 24: two row tiles; 40, 300: the
# large-M kernel (300: a ragged row block)
@pytest.mark.parametrize("bits,G,sym", VARIANTS)
@pytest.mark.parametrize("M", [1, 3, 8, 24, 40, 300])
def test_gemm_regimes(bits, G, sym, M):
    N, K = 224, 2560
    dtype = "bf16" if (M + bits) % 2 else "f16"
    act = M in (3, 8, 40) and G != -1
    say("bits gemm", bits, G, sym, M, dtype, act)
    tag = "gpu/bits/gemm/%d/%d/%d" % (bits, G, M)
    W = synth.weights(tag + "/W", N, K)
    gi = synth.act_order_gidx(tag + "/g", K, _g(K, G)) if act else None
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    _, packed = _pack(W, bits, G, gi, sym)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    err = compare_gemm(y, xb, _oracle_rows(W, bits, G, gi, sym, np.arange(N), dtype), dtype)
    say("  rel err", err)
    assert err <= TOL


@pytest.mark.parametrize("bits", [3, 8])
@pytest.mark.parametrize("M", [2, 16, 64])
def test_gemm_onehot_exact(bits, M):
    N, K, G = 128, 1024, 128
    dtype = "bf16" if M == 16 else "f16"
    say("bits onehot", bits, M)
    W = synth.weights("gpu/bits/oh/%d" % bits, N, K)
    gi = synth.act_order_gidx("gpu/bits/oh/g", K, G)
    _, packed = _pack(W, bits, G, gi, False)
    wd = _oracle_rows(W, bits, G, gi, False, np.arange(N), dtype)
    ks = (np.arange(M) * 131 + 7) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, dtype), dtype), packed))
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wd[:, k]), (r, k)


@pytest.mark.parametrize("bits", [3, 8])
@pytest.mark.parametrize("M", [2, 64])
def test_gemm_xscale(bits, M):
    N, K, G = 224, 2048, 128
    dtype = "bf16"
    say("bits xscale", bits, M)
    tag = "gpu/bits/xs/%d/%d" % (bits, M)
    W = synth.weights(tag + "/W", N, K)
    s32 = synth.awq_scales(tag + "/s", K)
    sb = synth.to_bits(s32[None, :], dtype)[0]
    Wf = (W.astype(np.float64) * fp.bits_to_f64(sb, dtype)[None, :]).astype(np.float32)
    _, packed = _pack(Wf, bits, G, None, False)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    y = w4.w4a16_gemm_xscale(bits_to_tensor(xb, dtype), bits_to_tensor(sb, dtype), packed)
    y_ref = gemm.gemm_ref_xscale_bits(xb, sb, _oracle_rows(Wf, bits, G, None, False,
                                                          np.arange(N), dtype), dtype)
    err = gemm.rel_err(tensor_f64(y, dtype), y_ref)
    say("  rel err", err)
    assert err <= TOL


@pytest.mark.parametrize("bits,M", [(3, 1), (8, 16)])
def test_gemm_large_layer_sampled(bits, M):
    # a layer of 100 Mi weights: M = 1 streams it through the decode kernel,
    # M = 16 runs the large-M kernel with a split of K; sampled columns
    N, K, G = 8192, 12800, 128
    dtype = "bf16"
    say("bits large layer", bits, M)
    tag = "gpu/bits/large/%d" % bits
    W = synth.weights(tag + "/W", N, K)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    _, packed = _pack(W, bits, G, None, False)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    rows = np.arange(11, N, 59)
    err = compare_gemm(y, xb, _oracle_rows(W, bits, G, None, False, rows, dtype), dtype, cols=rows)
    say("  rel err", err)
    assert err <= TOL
