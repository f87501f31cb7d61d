"""NF4 codes repacked into 1 KB tiles (nf4_repack): the device repack equals
the oracle's layout byte for byte, and nf4_gemm_repacked gives bitwise the
same output as nf4_gemm on the canonical codes (the same dequant and the same
accumulation order, only the code addresses differ) in every kernel form --
decode packed / full-row / transposed, one and two row tiles, the large-M
kernel with and without a split of K and its ragged-tail launch -- with a
ragged last K tile (K % 128 == 64, decode) and ragged N; and within the
tolerance of the oracle's product."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import nf4, gemm, repack
from gpu_util import DEV, say, bits_to_tensor, tensor_bits, compare_gemm

pytestmark = pytest.mark.gpu
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _packed(tag, N, K):
    W = synth.weights(tag, N, K)
    p = w4.nf4_quantize(torch.from_numpy(W).to(DEV), 64)
    return W, w4.nf4_repack(p)


@pytest.mark.parametrize("N,K", [(16, 128), (48, 320), (208, 1088), (256, 8192)])
def test_repack_bytes_equal_oracle(N, K):
    say("nf4 repack bytes", N, K)
    _, p = _packed("gpu/nf4r/bytes/%d/%d" % (N, K), N, K)
    torch.cuda.synchronize()
    want = repack.repack_nf4_ref(p["qweight"].cpu().numpy(), N, K)
    assert np.array_equal(p["qweight_r"].cpu().numpy(), want)


# (N, K, M): decode forms at K % 128 == 64 and == 0, the large-M kernel (K % 128 == 0)
CASES = [(208, 1088, M) for M in (1, 3, 4, 5, 8, 12, 16, 17, 32)] + \
        [(256, 4096, M) for M in (1, 4, 16, 24, 64, 70, 300)] + \
        [(28672, 8192, M) for M in (1, 32, 33)]


@pytest.mark.parametrize("N,K,M", CASES)
@pytest.mark.parametrize("dtype", ["bf16", "f16"])
def test_repacked_gemm_bitwise_equals_canonical(N, K, M, dtype):
    plan = w4.nf4_gemm_repacked_plan(M, N, K, dtype=TDT[dtype])
    say("nf4 repacked gemm", N, K, M, dtype, plan, "canonical", w4.nf4_gemm_plan(M, N, K,
                                                                                   dtype=TDT[dtype]))
    assert plan[0].startswith("w4a16::nf4r_decode_kernel") or ", 2, 1, 4>" in plan[0]
    _, p = _packed("gpu/nf4r/gemm/%d/%d" % (N, K), N, K)
    x = bits_to_tensor(synth.to_bits(synth.activations("gpu/nf4r/x/%d/%d" % (M, K), M, K), dtype),
                       dtype)
    canon = {k: v for k, v in p.items() if k != "qweight_r"}
    y_c = w4.nf4_gemm(x, canon)
    y_r = w4.nf4_gemm(x, p)
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(y_r), tensor_bits(y_c))


@pytest.mark.parametrize("M", [1, 16, 70])
def test_repacked_gemm_matches_oracle(M):
    N, K, dtype = 208, 1088 if M < 64 else 1024, "bf16"
    say("nf4 repacked vs oracle", N, K, M)
    W, p = _packed("gpu/nf4r/oracle/%d" % K, N, K)
    xb = synth.to_bits(synth.activations("gpu/nf4r/ox/%d" % M, M, K), dtype)
    y = w4.nf4_gemm(bits_to_tensor(xb, dtype), p)
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, dtype)
    assert compare_gemm(y, xb, wd, dtype) <= gemm.TOL
