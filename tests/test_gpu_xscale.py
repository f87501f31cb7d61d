"""GPU parity of w4a16_gemm_xscale (AWQ input scales applied by the GEMM)
against the oracle y = (x / s) w^T in fp64: within max|y - y_ref| / max|y_ref|
<= 5e-3 in every regime (scales fused into the decode kernels' loads; the
preparation pass with a permutation and for the large-M kernel), plus exact
cases: unit scales reproduce w4a16_gemm bit for bit, and power-of-two scales
on one-hot rows give exactly rounded single products."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import int4, gemm, fp
from gpu_util import DEV, say, bits_to_tensor, tensor_bits, tensor_f64

pytestmark = pytest.mark.gpu
TOL = gemm.TOL


def _awq_setup(tag, N, K, G, sym, act, dtype, s32=None):
    """AWQ-folded weights W' = W * s quantized on the device; s as 16-bit bits."""
    W = synth.weights(tag + "/W", N, K)
    if s32 is None:
        s32 = synth.awq_scales(tag + "/s", K)
    sb = synth.to_bits(s32[None, :], dtype)[0]
    sf = fp.bits_to_f64(sb, dtype)
    Wf = (W.astype(np.float64) * sf[None, :]).astype(np.float32)
    gi = synth.act_order_gidx(tag + "/g", K, G) if act else None
    Wd = torch.from_numpy(Wf).to(DEV)
    gid = torch.from_numpy(gi).to(DEV) if gi is not None else None
    qw, sc, qz = w4.w4a16_quantize_rtn(Wd, G, g_idx=gid, sym=sym)
    packed = w4.w4a16_repack(qw, sc, qz, gid, G)
    q, s, z = int4.quantize_rtn_int4(Wf, G, gi, sym=sym)
    wd = int4.dequant_codes(q, s, z, gi, G, dtype)            # original column order
    return packed, sb, wd


def _x(tag, M, K, dtype):
    x32 = synth.activations(tag + "/x", M, K)
    x32 = synth.with_outliers(x32, synth.outlier_channels(tag + "/o", K))
    return synth.to_bits(x32, dtype)


# M = 1, 3, 4: packed decode, scaled in its loads (3 with act-order: the
# preparation pass); 8, 20: full-row decode (8 with act-order: the pass);
# 40, 300: the large-M kernel behind the pass (300: a ragged row block)
@pytest.mark.parametrize("M", [1, 3, 4, 8, 20, 40, 300])
@pytest.mark.parametrize("G,sym", [(128, False), (64, True)])
def test_xscale_gemm_regimes(M, G, sym):
    N, K = 200, 2560
    dtype = "bf16" if (M + G) % 2 else "f16"
    act = M in (3, 8, 40)
    say("xscale gemm", M, G, sym, dtype, act)
    tag = "gpu/xs/%d/%d" % (M, G)
    packed, sb, wd = _awq_setup(tag, N, K, G, sym, act, dtype)
    xb = _x(tag, M, K, dtype)
    y = w4.w4a16_gemm_xscale(bits_to_tensor(xb, dtype), bits_to_tensor(sb, dtype), packed)
    torch.cuda.synchronize()
    y_ref = gemm.gemm_ref_xscale_bits(xb, sb, wd, dtype)
    err = gemm.rel_err(tensor_f64(y, dtype), y_ref)
    say("  rel err", err)
    assert err <= TOL


@pytest.mark.parametrize("M", [2, 16, 64])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_xscale_unit_scales_equal_plain_gemm(M, dtype):
    # x / 1 is x exactly (the reciprocal of 1 is exact): same bits as w4a16_gemm
    N, K, G = 256, 1024, 128
    say("xscale unit", M, dtype)
    tag = "gpu/xs/unit/%d" % M
    packed, sb, _ = _awq_setup(tag, N, K, G, False, False, dtype, np.ones(K, np.float32))
    x = bits_to_tensor(_x(tag, M, K, dtype), dtype)
    y1 = tensor_bits(w4.w4a16_gemm_xscale(x, bits_to_tensor(sb, dtype), packed))
    y2 = tensor_bits(w4.w4a16_gemm(x, packed))
    assert np.array_equal(y1, y2)


@pytest.mark.parametrize("M", [3, 12, 64])
@pytest.mark.parametrize("act", [False, True])
def test_xscale_onehot_power_of_two_exact(M, act):
    # s_k = 2^e_k and x_k = 1: x / s is a power of two, so a one-hot row
    # yields (x_k / s_k) * w[n, k] exactly, whether or not the kernel rounds
    # the dequantized weight to 16 bits before the product (its packed and
    # 32-row paths apply the scale after the K sum); a wrong channel's scale
    # shows as a different power of two
    N, K, G = 128, 1024, 128
    dtype = "f16"
    say("xscale onehot", M, act)
    r = np.random.default_rng(40 + M)
    s32 = (2.0 ** r.integers(-2, 3, size=K)).astype(np.float32)
    tag = "gpu/xs/oh/%d/%d" % (M, act)
    packed, sb, wd = _awq_setup(tag, N, K, G, False, act, dtype, s32)
    ks = (np.arange(M) * 97 + 5) % K
    x = np.zeros((M, K), dtype=np.float32)
    x[np.arange(M), ks] = 1.0
    xb = synth.to_bits(x, dtype)
    y = tensor_bits(w4.w4a16_gemm_xscale(bits_to_tensor(xb, dtype), bits_to_tensor(sb, dtype),
                                         packed))
    want = synth.to_bits(gemm.gemm_ref_xscale_bits(xb, sb, wd, dtype).astype(np.float32), dtype)
    assert np.array_equal(y, want)


def test_xscale_large_layer_sampled():
    # a layer of 100 Mi weights at M = 16: the large-M kernel with a split of
    # K, behind the preparation pass; sampled output columns
    N, K, G, M = 8192, 12800, 128, 16
    dtype = "bf16"
    say("xscale large layer")
    tag = "gpu/xs/large"
    W = synth.weights(tag + "/W", N, K)
    s32 = synth.awq_scales(tag + "/s", K)
    sb = synth.to_bits(s32[None, :], dtype)[0]
    sf = fp.bits_to_f64(sb, dtype)
    Wf = (W.astype(np.float64) * sf[None, :]).astype(np.float32)
    qw, sc, qz = w4.w4a16_quantize_rtn(torch.from_numpy(Wf).to(DEV), G)
    packed = w4.w4a16_repack(qw, sc, qz, None, G)
    xb = _x(tag, M, K, dtype)
    y = w4.w4a16_gemm_xscale(bits_to_tensor(xb, dtype), bits_to_tensor(sb, dtype), packed)
    torch.cuda.synchronize()
    rows = np.arange(5, N, 67)
    q, s, z = int4.quantize_rtn_int4(Wf[rows], G)
    wd = int4.dequant_codes(q, s, z, None, G, dtype)
    y_ref = gemm.gemm_ref_xscale_bits(xb, sb, wd, dtype)
    err = gemm.rel_err(tensor_f64(y, dtype)[:, rows], y_ref)
    say("  rel err", err)
    assert err <= TOL


@pytest.mark.parametrize("M", [3, 8, 40, 300])
@pytest.mark.parametrize("act", [False, True])
def test_xscale_gemm_without_workspace(M, act):
    # no workspace: no preparation pass; rows the decode kernel cannot stage on
    # chip are gathered (and divided by s) element by element from global
    # memory, at any M
    N, K = 200, 2560
    dtype = "bf16" if act else "f16"
    tag = "gpu/xs/nows/%d" % M
    say("xscale without workspace", M, act, dtype, w4.w4a16_gemm_plan(
        M, N, K, dtype=torch.bfloat16 if act else torch.float16, perm=act, x_scale=True,
        workspace=False))
    packed, sb, wd = _awq_setup(tag, N, K, 128, False, act, dtype)
    xb = _x(tag, M, K, dtype)
    y = w4.w4a16_gemm_xscale(bits_to_tensor(xb, dtype), bits_to_tensor(sb, dtype), packed,
                             use_workspace=False)
    torch.cuda.synchronize()
    y_ref = gemm.gemm_ref_xscale_bits(xb, sb, wd, dtype)
    err = gemm.rel_err(tensor_f64(y, dtype), y_ref)
    say("  rel err", err)
    assert err <= TOL
