"""GPU parity of the INT4 path against the oracle: quantizer, repack and dequant
bit-exact; GEMM within max|y - y_ref| / max|y_ref| <= 5e-3."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import int4, repack, gemm
from gpu_util import (DEV, say, bits_to_tensor, tensor_bits, tensor_f64, int4_inputs,
                      gpu_int4_pack, oracle_int4_rows, compare_gemm)

pytestmark = pytest.mark.gpu
TOL = gemm.TOL


@pytest.mark.parametrize("N,K,act", [(512, 512, False), (200, 384, False), (256, 1024, True),
                                     (72, 256, True)])
def test_quantizer_bit_exact(N, K, act):
    say("quantizer", N, K, act)
    W, gi, _ = int4_inputs("gpu/quant/%d/%d" % (N, K), N, K, act_order=act)
    (qw, sc, qz), _ = gpu_int4_pack(W, gi)
    q, s, z = int4.quantize_rtn_int4(W, 128, gi)
    assert np.array_equal(qw.cpu().numpy(), int4.pack_qweight(q))
    assert np.array_equal(tensor_bits(sc), s.view(np.uint16))
    assert np.array_equal(qz.cpu().numpy(), int4.pack_qzeros(z))


@pytest.mark.parametrize("N,K,act", [(512, 512, False), (200, 384, True), (1024, 256, True)])
def test_repack_bytes_equal_reference(N, K, act):
    say("repack", N, K, act)
    W, gi, _ = int4_inputs("gpu/repack/%d/%d" % (N, K), N, K, act_order=act)
    (qw, sc, qz), packed = gpu_int4_pack(W, gi)
    ref = repack.repack_ref(qw.cpu().numpy(), sc.cpu().numpy(), qz.cpu().numpy(), gi)
    assert np.array_equal(packed["codes"].cpu().numpy(), ref[0])
    assert np.array_equal(tensor_bits(packed["scales"]), ref[1].view(np.uint16))
    assert np.array_equal(packed["zeros"].cpu().numpy().view(np.uint32), ref[2])
    if ref[3] is None:
        assert packed["perm"] is None
    else:
        assert np.array_equal(packed["perm"].cpu().numpy(), ref[3])


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
@pytest.mark.parametrize("act", [False, True])
def test_dequant_bit_exact(dtype, act):
    N, K = 264, 512
    say("dequant", dtype, act)
    W, gi, _ = int4_inputs("gpu/deq/%s" % dtype, N, K, act_order=act)
    _, packed = gpu_int4_pack(W, gi)
    got = tensor_bits(w4.w4a16_dequant(packed, torch.float16 if dtype == "f16" else torch.bfloat16))
    want = oracle_int4_rows(W, gi, np.arange(N), dtype)
    perm = repack.canonical_perm(gi, K)
    if perm is not None:
        want = want[:, perm]
    assert np.array_equal(got, want)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dequant_special_scales_bit_exact(dtype):
    # all 256 (q, z) pairs against powers of two, fp16 subnormals, large scales
    N, K = 64, 16 * 128
    r = np.random.default_rng(11)
    q = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))
    z = (np.arange(K // 128)[:, None] + np.arange(N)[None, :]) % 16
    svals = np.array([2.0**-24, 3 * 2.0**-24, 2.0**-15, 0.5, 1.0, 3.0, 1024.0, 4095.0,
                      60000.0, 2.0**-14, 1e-3, 0.0071, 7.0e-5, 2.0, 0.25, 65504.0], np.float16)
    s = svals[(np.arange(K // 128)[:, None] * 7 + np.arange(N)[None, :]) % 16]
    s = np.where(r.random(s.shape) < 0.2, -s, s).astype(np.float16)
    qw = torch.from_numpy(int4.pack_qweight(q)).to(DEV)
    sc = torch.from_numpy(s.view(np.int16)).view(torch.float16).to(DEV)
    qz = torch.from_numpy(int4.pack_qzeros(z.astype(np.uint8))).to(DEV)
    packed = w4.w4a16_repack(qw, sc, qz)
    got = tensor_bits(w4.w4a16_dequant(packed, torch.float16 if dtype == "f16" else torch.bfloat16))
    want = int4.dequant_int4(int4.pack_qweight(q), s, int4.pack_qzeros(z.astype(np.uint8)), None,
                             128, dtype)
    assert np.array_equal(got, want)


def _run_gemm(tag, M, N, K, dtype, act=False, awq=False, xscale=1.0):
    W, gi, s = int4_inputs(tag, N, K, act_order=act, awq=awq)
    x32 = synth.activations(tag + "/x", M, K) * np.float32(xscale)
    if awq:
        x32 = (x32 / s[None, :]).astype(np.float32)
    xb = synth.to_bits(x32, dtype)
    _, packed = gpu_int4_pack(W, gi)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
    torch.cuda.synchronize()
    return y, xb, W, gi, packed


@pytest.mark.parametrize("M", [1, 2, 3, 4, 7, 8, 15, 16, 17, 31, 32, 33, 63, 64, 65, 130])
def test_gemm_m_sweep_f16(M):
    N, K = 200, 512                         # ragged N: one zero-padded panel
    say("gemm f16 M", M)
    y, xb, W, gi, _ = _run_gemm("gpu/gemm/msweep/%d" % M, M, N, K, "f16")
    wd = oracle_int4_rows(W, gi, np.arange(N), "f16")
    assert compare_gemm(y, xb, wd, "f16") <= TOL


@pytest.mark.parametrize("M", [1, 16, 33, 64, 100])
@pytest.mark.parametrize("act", [False, True])
def test_gemm_bf16_and_act_order(M, act):
    N, K = 256, 1024
    say("gemm bf16 M", M, "act", act)
    y, xb, W, gi, _ = _run_gemm("gpu/gemm/bf16/%d/%d" % (M, act), M, N, K, "bf16", act=act)
    wd = oracle_int4_rows(W, gi, np.arange(N), "bf16")
    assert compare_gemm(y, xb, wd, "bf16") <= TOL


def test_gemm_config1_tiny():
    # x fp16 [16, 512] ~ N(0,1); W [512, 512] ~ N(0, 0.02) RTN G=128; y fp16
    say("config 1 tiny")
    y, xb, W, gi, _ = _run_gemm("C1", 16, 512, 512, "f16")
    wd = oracle_int4_rows(W, gi, np.arange(512), "f16")
    err = compare_gemm(y, xb, wd, "f16")
    say("config 1 rel err", err)
    assert err <= TOL


@pytest.mark.parametrize("act", [True, False])
def test_gemm_long_k_sampled_columns(act):
    M, N, K = 4, 1024, 4096
    say("long K", act)
    y, xb, W, gi, _ = _run_gemm("gpu/gemm/split", M, N, K, "f16", act=act)
    rows = np.arange(0, N, 7)
    wd = oracle_int4_rows(W, gi, rows, "f16")
    assert compare_gemm(y, xb, wd, "f16", cols=rows) <= TOL


def test_gemm_perm_requires_workspace():
    # M > 4: the activations are permuted into the workspace first
    W, gi, _ = int4_inputs("gpu/gemm/nows", 64, 256, act_order=True)
    _, packed = gpu_int4_pack(W, gi)
    x = bits_to_tensor(synth.to_f16_bits(synth.activations("gpu/gemm/nows/x", 8, 256)), "f16")
    with pytest.raises(w4.W4A16Error):
        w4.w4a16_gemm(x, packed, use_workspace=False)


@pytest.mark.parametrize("M,K", [(1, 512), (2, 1024), (3, 2048), (4, 4096), (1, 11008),
                                 (4, 11008)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_act_order_small_m(M, K, dtype):
    # M <= 4: the kernel gathers x[:, perm] from on-chip staging without a
    # workspace when it fits (the last case does not: permuted through the
    # workspace); sampled columns at the larger K
    N = 96
    say("act-order small M", M, K, dtype)
    W, gi, _ = int4_inputs("gpu/gemm/gather/%d" % K, N, K, act_order=True)
    xb = synth.to_bits(synth.activations("gpu/gemm/gather/x/%d/%d" % (M, K), M, K), dtype)
    _, packed = gpu_int4_pack(W, gi)
    need = w4.w4a16_workspace_bytes(M, N, K)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed, use_workspace=need > 0)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    assert compare_gemm(y, xb, wd, dtype) <= TOL


def test_gemm_deterministic_and_scaling_exact():
    M, N, K = 16, 512, 2048
    say("determinism")
    W, gi, _ = int4_inputs("gpu/gemm/det", N, K, act_order=True)
    x32 = synth.activations("gpu/gemm/det/x", M, K)
    xb = synth.to_f16_bits(x32)
    # exact doubling of the fp16 inputs (doubling before rounding would differ
    # for fp16-subnormal inputs)
    x2b = synth.to_f16_bits(2 * xb.view(np.float16).astype(np.float32))
    _, packed = gpu_int4_pack(W, gi)
    y1 = tensor_bits(w4.w4a16_gemm(bits_to_tensor(xb, "f16"), packed))
    y2 = tensor_bits(w4.w4a16_gemm(bits_to_tensor(xb, "f16"), packed))
    assert np.array_equal(y1, y2)
    y3 = w4.w4a16_gemm(bits_to_tensor(x2b, "f16"), packed).float().cpu().numpy()
    y1f = y1.view(np.float16).astype(np.float32)
    # doubling is exact through the fp32 accumulation; the final fp16 rounding
    # commutes with it except in the fp16 subnormal range (absolute step 2^-24)
    normal = np.abs(y1f) >= 2.0**-14
    bad = np.nonzero(normal & (y3 != 2 * y1f))
    assert bad[0].size == 0, list(zip(bad[0][:5], bad[1][:5], y1f[bad][:5], y3[bad][:5]))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_onehot_reads_dequantized_weight_exactly(dtype):
    N, K = 128, 512
    say("onehot", dtype)
    W, gi, _ = int4_inputs("gpu/onehot", N, K, act_order=True)
    _, packed = gpu_int4_pack(W, gi)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    ks = [0, 1, 127, 128, 300, 511]
    x = np.zeros((len(ks), K), dtype=np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, dtype), dtype), packed))
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], wd[:, k]), k


def test_gemm_q_equals_z_gives_zero():
    M, N, K = 5, 128, 256
    z = np.random.default_rng(12).integers(0, 16, size=(K // 128, N)).astype(np.uint8)
    q = z[np.arange(K) // 128].T.copy()
    s = np.full((K // 128, N), 0.01, dtype=np.float16)
    packed = w4.w4a16_repack(torch.from_numpy(int4.pack_qweight(q)).to(DEV),
                             torch.from_numpy(s.view(np.int16)).view(torch.float16).to(DEV),
                             torch.from_numpy(int4.pack_qzeros(z)).to(DEV))
    x = bits_to_tensor(synth.to_f16_bits(synth.activations("gpu/qz/x", M, K)), "f16")
    y = w4.w4a16_gemm(x, packed)
    assert not torch.any(y.view(torch.int16) & 0x7FFF)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_subnormal_activation_is_not_flushed(dtype):
    # one-hot rows whose single nonzero is the smallest subnormal of the input
    # type, against a weight column of large exact values: y = x * w is exact
    # and far from underflow in the output, so a flushed input shows as 0.
    N, K = 64, 256
    q = np.full((N, K), 15, dtype=np.uint8)
    z = np.zeros((K // 128, N), dtype=np.uint8)
    s = np.full((K // 128, N), 1024.0, dtype=np.float16)       # w = 15 * 1024
    packed = w4.w4a16_repack(torch.from_numpy(int4.pack_qweight(q)).to(DEV),
                             torch.from_numpy(s.view(np.int16)).view(torch.float16).to(DEV),
                             torch.from_numpy(int4.pack_qzeros(z)).to(DEV))
    tiny = np.uint16(0x0001)                                    # smallest subnormal
    xb = np.zeros((2, K), dtype=np.uint16)
    xb[0, 3] = tiny
    xb[1, 200] = tiny | 0x8000
    y = tensor_f64(w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed), dtype)
    sub = 2.0**-24 if dtype == "f16" else 2.0**-133
    want = 15 * 1024.0 * sub          # 1.875 * 2^e: exact in both output types
    assert np.all(y[0] == want), y[0][:4]
    assert np.all(y[1] == -want)


@pytest.mark.parametrize("M,N,K", [(6, 160, 1024), (12, 160, 1024), (16, 4112, 512), (24, 208, 2048)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_full_row_modes_onehot_exact(M, N, K, dtype):
    # the decode kernel's full-row modes, act-order: direct loads (6 rows on
    # 160 columns) and whole-line loads through the LDS transpose (12, 16 on
    # 4112 columns, 24 rows in two row tiles).  One nonzero 1.0 per row puts
    # one dequantized weight in each output: any misplaced chunk of the
    # transpose shows as a wrong value
    say("full-row onehot", M, N, K, dtype)
    W, gi, _ = int4_inputs("gpu/gemm/fullrow/%d/%d" % (N, K), N, K, act_order=True)
    _, packed = gpu_int4_pack(W, gi)
    ks = (np.arange(M) * 37 + 5) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    y = tensor_bits(w4.w4a16_gemm(bits_to_tensor(synth.to_bits(x, dtype), dtype), packed))
    cols = np.unique(np.concatenate([np.arange(0, N, 7), [N - 1]]))
    wd = oracle_int4_rows(W, gi, cols, dtype)
    for r, k in enumerate(ks):
        assert np.array_equal(y[r][cols], wd[:, k]), (r, k)
