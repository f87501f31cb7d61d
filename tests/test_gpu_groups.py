"""GPU parity of the INT4 format variants against the oracle: group sizes 32,
64, multiples of 128 and per-channel (G = K, passed as -1), with asymmetric or
symmetric codes.  Quantizer, repack and dequant are compared bit for bit; the
GEMM within max|y - y_ref| / max|y_ref| <= 5e-3 in every kernel regime
(packed, gathered and full-row decode; the large-M kernel with and without a
split of K)."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import int4, repack, gemm
from gpu_util import DEV, say, bits_to_tensor, tensor_bits, compare_gemm

pytestmark = pytest.mark.gpu
TOL = gemm.TOL
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}

# (group_size, symmetric)
VARIANTS = [(32, False), (32, True), (64, False), (64, True), (256, False), (-1, True),
            (128, True)]


def _g(K, G):
    return K if G == -1 else G


def _inputs(tag, N, K, G, act):
    W = synth.weights(tag + "/W", N, K)
    gi = synth.act_order_gidx(tag + "/g", K, _g(K, G)) if act else None
    return W, gi


def _pack(W, G, gi, sym):
    Wd = torch.from_numpy(W).to(DEV)
    gid = torch.from_numpy(gi).to(DEV) if gi is not None else None
    qw, sc, qz = w4.w4a16_quantize_rtn(Wd, G, g_idx=gid, sym=sym)
    packed = w4.w4a16_repack(qw, sc, qz, gid, G)
    return (qw, sc, qz), packed


def _oracle_rows(W, G, gi, sym, rows, dtype):
    K = W.shape[1]
    q, s, z = int4.quantize_rtn_int4(W[rows], _g(K, G), gi, sym=sym)
    return int4.dequant_codes(q, s, z, gi, _g(K, G), dtype)


@pytest.mark.parametrize("G,sym", VARIANTS)
@pytest.mark.parametrize("act", [False, True])
def test_quantizer_and_repack_bit_exact(G, sym, act):
    N, K = 200, 1024
    say("variant quantizer+repack", G, sym, act)
    W, gi = _inputs("gpu/var/q/%d/%d" % (G, sym), N, K, G, act)
    (qw, sc, qz), packed = _pack(W, G, gi, sym)
    q, s, z = int4.quantize_rtn_int4(W, _g(K, G), gi, sym=sym)
    assert np.array_equal(qw.cpu().numpy(), int4.pack_qweight(q))
    assert np.array_equal(tensor_bits(sc), s.view(np.uint16))
    assert (qz is None) == sym
    if not sym:
        assert np.array_equal(qz.cpu().numpy(), int4.pack_qzeros(z))
    ref = repack.repack_ref(int4.pack_qweight(q), s, None if sym else int4.pack_qzeros(z), gi,
                            _g(K, G))
    assert np.array_equal(packed["codes"].cpu().numpy(), ref[0])
    assert np.array_equal(tensor_bits(packed["scales"]), ref[1].view(np.uint16))
    if sym:
        assert packed["zeros"] is None and ref[2] is None
    else:
        assert np.array_equal(packed["zeros"].cpu().numpy().view(np.uint32), ref[2])
    if ref[3] is None:
        assert packed["perm"] is None
    else:
        assert np.array_equal(packed["perm"].cpu().numpy(), ref[3])


@pytest.mark.parametrize("G,sym", VARIANTS)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dequant_bit_exact(G, sym, dtype):
    N, K = 136, 2560                      # 20 K tiles: two full runs of 8 and a partial one
    say("variant dequant", G, sym, dtype)
    act = G in (32, 256)
    W, gi = _inputs("gpu/var/deq/%d/%d" % (G, sym), N, K, G, act)
    _, packed = _pack(W, G, gi, sym)
    got = tensor_bits(w4.w4a16_dequant(packed, TDT[dtype]))
    want = _oracle_rows(W, G, gi, sym, np.arange(N), dtype)
    perm = repack.canonical_perm(gi, K, _g(K, G))
    if perm is not None:
        want = want[:, perm]
    assert np.array_equal(got, want)


# M = 1, 3: packed decode (3 with act-order: gathered from LDS); 8: full-row
# decode (with act-order: x permuted through the workspace); 24: two row
# tiles; 40, 300: the large-M kernel (300: a ragged row block)
@pytest.mark.parametrize("G,sym", VARIANTS)
@pytest.mark.parametrize("M", [1, 3, 8, 24, 40, 300])
def test_gemm_regimes(G, sym, M):
    N, K = 200, 2560
    dtype = "bf16" if (M + _g(K, G)) % 2 else "f16"
    act = M in (3, 8, 40) and G != -1
    say("variant gemm", G, sym, M, dtype, act)
    tag = "gpu/var/gemm/%d/%d/%d" % (G, sym, M)
    W, gi = _inputs(tag, N, K, G, act)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    _, packed = _pack(W, G, gi, sym)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    wd = _oracle_rows(W, G, gi, sym, np.arange(N), dtype)
    err = compare_gemm(y, xb, wd, dtype)
    say("  rel err", err)
    assert err <= TOL


@pytest.mark.parametrize("G,sym", [(32, True), (64, False), (-1, False)])
@pytest.mark.parametrize("M", [2, 16, 64])
def test_gemm_onehot_exact(G, sym, M):
    # one-hot activation rows read single dequantized weights: exact outputs
    N, K = 128, 1024
    dtype = "bf16" if M == 16 else "f16"
    say("variant onehot", G, sym, M)
    W, gi = _inputs("gpu/var/onehot/%d" % G, N, K, G, G == 32)
    _, packed = _pack(W, G, gi, sym)
    wd = _oracle_rows(W, G, gi, sym, np.arange(N), dtype)
    ks = (np.arange(M) * 131 + 7) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, dtype), dtype), packed))
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wd[:, k]), (r, k)


@pytest.mark.parametrize("G,sym,M", [(32, True, 64), (64, False, 16)])
def test_gemm_large_layer_split_k_sampled(G, sym, M):
    # a layer of 100 Mi weights: M = 16 runs the large-M kernel there, and both
    # M split K over workgroups; sampled output columns against the oracle
    N, K = 8192, 12800
    dtype = "bf16"
    say("variant large layer", G, sym, M)
    tag = "gpu/var/large/%d/%d" % (G, M)
    W, gi = _inputs(tag, N, K, G, False)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    _, packed = _pack(W, G, gi, sym)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    rows = np.arange(3, N, 61)
    wd = _oracle_rows(W, G, gi, sym, rows, dtype)
    err = compare_gemm(y, xb, wd, dtype, cols=rows)
    say("  rel err", err)
    assert err <= TOL
