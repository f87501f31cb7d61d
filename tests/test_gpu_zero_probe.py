"""The zero probe on every kernel path: weights whose every code equals its
group's zero point (q == z, so (q - z) s = 0 for every weight) give y == 0
exactly, whatever the activations; NF4 weights whose every code is the zero
level (L[7] = 0) likewise.

This is the special case in which the dequantized weight matrix is exactly
zero ([P3] §2.1: the zero point is the code of the real value 0), so the
product must be exactly zero on every path -- including the ones that apply
the scale and zero after a K tile's sum, s * (sum x (o + q) - sum x (o + z)),
where it holds only because both sums come from identical MFMA inputs.  The
activations carry large outlier channels so that the two sums are large and
any difference between them would show.

Paths (the plan query names each call's kernels in the test output): the
decode kernel's packed modes (M <= 4; act-order rows gathered on chip, AWQ
input scales staged on chip, the wide two-tile kernel on >= 16384 columns),
its full-row modes (M = 5..8 direct, M = 12 and 16 transposed, with the fold
at G >= 128), the large-M kernel's 32-row tiles (with the fold) and 64-row
tiles, with and without a split of K, and the no-workspace forms (the global
gather).
"""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import intb
from gpu_util import DEV, say, bits_to_tensor, tensor_bits

pytestmark = pytest.mark.gpu


def _zero_weight(tag, N, K, bits, G, sym, act):
    """Canonical tensors with q == z everywhere: zeros (or the implicit zero of
    a symmetric weight) per (column, group), every code of the group equal to
    it; random fp16 scales of both signs over many binades."""
    g = K if G == -1 else G
    r = synth.rng(tag)
    gi = synth.act_order_gidx(tag + "/g", K, g) if act else None
    grp = gi if gi is not None else (np.arange(K) // g)
    if sym:
        z = np.full((K // g, N), intb.sym_zero(bits), dtype=np.uint8)
    else:
        z = r.integers(0, 1 << bits, size=(K // g, N)).astype(np.uint8)
    q = np.ascontiguousarray(z[grp, :].T)                      # [N, K]
    mag = np.exp2(r.uniform(-14, 4, size=(K // g, N)))
    s = (mag * np.where(r.random((K // g, N)) < 0.3, -1.0, 1.0)).astype(np.float16)
    qw = torch.from_numpy(intb.pack_qweight(q, bits).view(np.int32)).to(DEV)
    sc = torch.from_numpy(s.view(np.int16)).view(torch.float16).to(DEV)
    qz = None if sym else torch.from_numpy(intb.pack_qzeros(z, bits).view(np.int32)).to(DEV)
    gid = torch.from_numpy(gi).to(DEV) if gi is not None else None
    return w4.w4a16_repack(qw, sc, qz, gid, G, bits=bits)


def _x(tag, M, K, dtype):
    x32 = synth.with_outliers(synth.activations(tag, M, K), synth.outlier_channels(tag + "/oc", K))
    x32[:, :: max(1, K // 5)] *= np.float32(2.0 ** (8 if dtype == "f16" else 40))
    return bits_to_tensor(synth.to_bits(x32, dtype), dtype)


def _assert_zero(y, what):
    b = tensor_bits(y)
    nz = np.count_nonzero(b & 0x7FFF)
    assert nz == 0, "%s: %d nonzero outputs, e.g. %s" % (what, nz, b[b & 0x7FFF != 0][:4])


TDT = {"f16": torch.float16, "bf16": torch.bfloat16}
# (bits, G, sym, act-order)
CASES = [(4, 128, False, False), (4, 128, False, True), (4, 32, False, True), (4, 64, True, False),
         (4, -1, False, False), (3, 128, False, False), (3, 32, False, True),
         (8, 128, False, False), (8, 64, True, True)]


@pytest.mark.parametrize("bits,G,sym,act", CASES)
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_codes_give_zero_every_m(bits, G, sym, act, dtype):
    N, K = 256, 1024
    tag = "gpu/zero/%d/%d/%d/%d" % (bits, G, sym, act)
    packed = _zero_weight(tag, N, K, bits, G, sym, act)
    for M in (1, 2, 3, 4, 5, 8, 12, 16, 32, 33, 64):
        for ws in (True, False):
            plan = w4.w4a16_gemm_plan(M, N, K, G, bits, TDT[dtype], perm=packed["perm"] is not None,
                                      workspace=ws)
            say("zero probe", bits, G, sym, act, dtype, "M", M, "ws", ws, plan)
            y = w4.w4a16_gemm(_x(tag + "/x/%d" % M, M, K, dtype), packed, use_workspace=ws)
            torch.cuda.synchronize()
            _assert_zero(y, "M=%d ws=%s %s" % (M, ws, plan))


@pytest.mark.parametrize("bits,G,sym", [(4, 128, False), (3, 32, False), (8, 64, True)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_codes_give_zero_wide_layer(bits, G, sym, dtype):
    # >= 16384 columns: the wide two-tile packed kernel at 3 and 4 rows
    N, K = 16416, 512
    tag = "gpu/zero/wide/%d/%d" % (bits, G)
    packed = _zero_weight(tag, N, K, bits, G, sym, False)
    for M in (1, 3, 4, 12):
        plan = w4.w4a16_gemm_plan(M, N, K, G, bits, TDT[dtype])
        say("zero probe wide", bits, G, dtype, "M", M, plan)
        y = w4.w4a16_gemm(_x(tag + "/x/%d" % M, M, K, dtype), packed)
        torch.cuda.synchronize()
        _assert_zero(y, "M=%d %s" % (M, plan))


@pytest.mark.parametrize("G,act", [(128, False), (32, True), (128, True)])
@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_codes_give_zero_with_input_scales(G, act, dtype):
    # AWQ input scales: staged and divided on chip (M <= 4), the preparation
    # pass (with a workspace) or the global gather (without)
    N, K = 256, 1024
    tag = "gpu/zero/xs/%d/%d" % (G, act)
    packed = _zero_weight(tag, N, K, 4, G, False, act)
    s = bits_to_tensor(synth.to_bits(synth.awq_scales(tag + "/s", K)[None, :], dtype)[0], dtype)
    for M in (1, 4, 12, 33):
        for ws in (True, False):
            plan = w4.w4a16_gemm_plan(M, N, K, G, 4, TDT[dtype], perm=act, x_scale=True,
                                      workspace=ws)
            say("zero probe xscale", G, act, dtype, "M", M, "ws", ws, plan)
            y = w4.w4a16_gemm_xscale(_x(tag + "/x/%d" % M, M, K, dtype), s, packed,
                                     use_workspace=ws)
            torch.cuda.synchronize()
            _assert_zero(y, "M=%d ws=%s %s" % (M, ws, plan))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_zero_codes_give_zero_large_layer_tiles(dtype):
    # 24 Mi weights with N < 5120: the large-M kernel's 32-row tiles from 17
    # rows, with a partial row block (M = 20) and a whole one (M = 32)
    N, K = 4096, 6144
    tag = "gpu/zero/large"
    packed = _zero_weight(tag, N, K, 4, 128, False, True)
    for M in (16, 20, 32):
        plan = w4.w4a16_gemm_plan(M, N, K, 128, 4, TDT[dtype], perm=True)
        say("zero probe large", dtype, "M", M, plan)
        y = w4.w4a16_gemm(_x(tag + "/x/%d" % M, M, K, dtype), packed)
        torch.cuda.synchronize()
        _assert_zero(y, "M=%d %s" % (M, plan))


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_nf4_zero_level_gives_zero(dtype):
    # every code 7 (the level 0.0) with random double-quantized absmax
    N, K = 256, 2048
    r = synth.rng("gpu/zero/nf4")
    nf = {"qweight": torch.full((N, K // 2), 0x77, dtype=torch.uint8, device=DEV),
          "absmax_q": torch.from_numpy(r.integers(0, 256, size=N * K // 64).astype(np.uint8)).to(DEV),
          "absmax_scale": torch.from_numpy(r.uniform(1e-4, 1.0, size=(N * K // 64 + 255) // 256)
                                           .astype(np.float32)).to(DEV),
          "N": N, "K": K, "blocksize": 64}
    for M in (1, 4, 12, 16, 32, 33, 64):
        for ws in (True, False):
            plan = w4.nf4_gemm_plan(M, N, K, 64, TDT[dtype], workspace=ws)
            say("zero probe nf4", dtype, "M", M, "ws", ws, plan)
            y = w4.nf4_gemm(_x("gpu/zero/nf4/x/%d" % M, M, K, dtype), nf, use_workspace=ws)
            torch.cuda.synchronize()
            _assert_zero(y, "M=%d ws=%s %s" % (M, ws, plan))
