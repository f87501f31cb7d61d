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


@pytest.mark.parametrize("M", [1, 4, 5, 8, 16, 33, 64, 130])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_gemm_act_order_without_workspace(M, dtype):
    # no workspace: no preparation pass; the decode kernel gathers x[m][perm[k]]
    # itself (on chip for M <= 4 where the rows fit, else from global memory,
    # at any M) -- the same product as the call with a workspace
    N, K = 200, 1024
    say("act-order without workspace", M, dtype, w4.w4a16_gemm_plan(
        M, N, K, dtype=torch.float16 if dtype == "f16" else torch.bfloat16, perm=True,
        workspace=False))
    W, gi, _ = int4_inputs("gpu/gemm/nows/%d" % M, N, K, act_order=True)
    _, packed = gpu_int4_pack(W, gi)
    xb = synth.to_bits(synth.activations("gpu/gemm/nows/x/%d" % M, M, K), dtype)
    y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed, use_workspace=False)
    torch.cuda.synchronize()
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)       # original column order
    assert compare_gemm(y, xb, wd, dtype) <= TOL


@pytest.mark.parametrize("M", [32, 64, 200])
def test_gemm_large_m_without_workspace_no_split(M):
    # the large-M kernel without a workspace: no split of K (the plan with a
    # workspace splits K over workgroups on this narrow layer)
    N, K = 256, 4096
    with_ws = w4.w4a16_gemm_plan(M, N, K, dtype=torch.bfloat16)
    without = w4.w4a16_gemm_plan(M, N, K, dtype=torch.bfloat16, workspace=False)
    say("large M without workspace", M, with_ws, without)
    assert not any("split_reduce" in k for k in without)
    W, gi, _ = int4_inputs("gpu/gemm/nows/pf/%d" % M, N, K)
    _, packed = gpu_int4_pack(W, gi)
    xb = synth.to_bits(synth.activations("gpu/gemm/nows/pf/x/%d" % M, M, K), "bf16")
    y0 = w4.w4a16_gemm(bits_to_tensor(xb, "bf16"), packed, use_workspace=False)
    y1 = w4.w4a16_gemm(bits_to_tensor(xb, "bf16"), packed)
    torch.cuda.synchronize()
    wd = oracle_int4_rows(W, gi, np.arange(N), "bf16")
    assert compare_gemm(y0, xb, wd, "bf16") <= TOL
    assert compare_gemm(y1, xb, wd, "bf16") <= TOL


@pytest.mark.parametrize("M", list(range(1, 18)) + [63, 64, 65])
@pytest.mark.parametrize("act", [False, True])
def test_gemm_m_sweep_bf16_every_small_m(M, act):
    # every M from 1 to 17 (the decode forms: packed, staged gather, one-row
    # fold, full rows, transposed rows, the operand layout after the pass,
    # two row tiles at 17) and 63-65 (row tiles / large-M block edges), with
    # and without act-order, K with 5 K tiles (a partial run of 8) and ragged N
    N, K = 208, 640
    say("gemm bf16 sweep M", M, "act", act, w4.w4a16_gemm_plan(M, N, K, dtype=torch.bfloat16,
                                                                 perm=act))
    y, xb, W, gi, _ = _run_gemm("gpu/gemm/sweep/%d/%d" % (M, act), M, N, K, "bf16", act=act)
    wd = oracle_int4_rows(W, gi, np.arange(N), "bf16")
    assert compare_gemm(y, xb, wd, "bf16") <= TOL
