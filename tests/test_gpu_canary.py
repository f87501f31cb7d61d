"""Out-of-bounds write detection: every kernel family writes only inside its
output [M, N] and inside the workspace bytes the library asked for.  The
output and the workspace sit between guard regions filled with a known
pattern, on ragged shapes (M and N not multiples of the tiles, N = 200 or
208: a partly filled last panel of 64 columns); after each call the guards
must be untouched and the output must match the oracle.

Paths (the plan query names each call's kernels in the test output): decode
packed / full-row / transposed modes, the wide two-tile kernel, the
preparation pass (act-order and AWQ scales), the large-M kernel with whole
and partial row blocks, its split of K with split_reduce_kernel, NF4 decode
and large-M."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import gemm, nf4
from gpu_util import DEV, say, bits_to_tensor, int4_inputs, gpu_int4_pack, oracle_int4_rows, \
    compare_gemm

pytestmark = pytest.mark.gpu
TOL = gemm.TOL
GUARD = 8192                       # bytes of guard on each side (keeps 16-byte alignment)
PAT = 0xA5


def _guarded(nbytes):
    """A uint8 device buffer [guard | nbytes | guard] filled with the pattern,
    and the middle view."""
    buf = torch.full((2 * GUARD + max(nbytes, 16),), PAT, dtype=torch.uint8, device=DEV)
    return buf, buf[GUARD:GUARD + nbytes]


def _check_guards(buf, nbytes, what):
    b = buf.cpu().numpy()
    lo, hi = b[:GUARD], b[GUARD + max(nbytes, 16):]
    bad = np.count_nonzero(lo != PAT) + np.count_nonzero(hi != PAT)
    assert bad == 0, "%s: %d guard bytes overwritten (before: %s, after: %s)" % (
        what, bad, np.nonzero(lo != PAT)[0][-4:], np.nonzero(hi != PAT)[0][:4])


TDT = {"f16": torch.float16, "bf16": torch.bfloat16}

# (M, N, K, act-order, AWQ input scales, dtype)
INT_CASES = [(1, 200, 1024, False, False, "f16"), (3, 200, 1024, True, False, "bf16"),
             (4, 200, 1024, False, True, "f16"), (5, 200, 1024, False, False, "bf16"),
             (12, 200, 1024, True, False, "f16"), (17, 200, 1024, False, False, "bf16"),
             (33, 200, 1024, True, False, "bf16"), (64, 200, 4096, False, False, "f16"),
             (130, 200, 1024, False, True, "bf16"), (3, 16400, 512, False, False, "f16"),
             (300, 208, 2048, True, False, "f16")]


@pytest.mark.parametrize("M,N,K,act,xs,dtype", INT_CASES)
def test_int4_writes_stay_inside_output_and_workspace(M, N, K, act, xs, dtype):
    tag = "gpu/canary/%d/%d/%d" % (M, N, K)
    plan = w4.w4a16_gemm_plan(M, N, K, dtype=TDT[dtype], perm=act, x_scale=xs)
    say("canary int4", M, N, K, act, xs, dtype, plan)
    W, gi, s = int4_inputs(tag, N, K, act_order=act, awq=xs)
    _, packed = gpu_int4_pack(W, gi)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    obuf, ov = _guarded(2 * M * N)
    out = ov.view(TDT[dtype]).view(M, N)
    need = w4.w4a16_workspace_bytes(M, N, K)
    wbuf, wv = _guarded(need)
    ws = wv if need > 0 else None
    x = bits_to_tensor(xb, dtype)
    if xs:
        sb = synth.to_bits(s[None, :], dtype)[0]
        w4.w4a16_gemm_xscale(x, bits_to_tensor(sb, dtype), packed, out=out, workspace=ws)
    else:
        w4.w4a16_gemm(x, packed, out=out, workspace=ws)
    torch.cuda.synchronize()
    _check_guards(obuf, 2 * M * N, "output")
    _check_guards(wbuf, need, "workspace")
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    if xs:
        y_ref = gemm.gemm_ref_xscale_bits(xb, synth.to_bits(s[None, :], dtype)[0], wd, dtype)
        from gpu_util import tensor_f64
        assert gemm.rel_err(tensor_f64(out, dtype), y_ref) <= TOL
    else:
        assert compare_gemm(out, xb, wd, dtype) <= TOL


def test_split_reduce_case_is_in_the_list():
    # the canary cases include a large-M call that splits K (split_reduce_kernel)
    assert any(k.startswith("w4a16::split_reduce_kernel")
               for k in w4.w4a16_gemm_plan(64, 200, 4096, dtype=torch.float16))


@pytest.mark.parametrize("M,N,K", [(1, 208, 1024), (12, 208, 2048), (33, 208, 2048),
                                   (64, 208, 4096)])
def test_nf4_writes_stay_inside_output_and_workspace(M, N, K):
    plan = w4.nf4_gemm_plan(M, N, K)
    say("canary nf4", M, N, K, plan)
    W = synth.weights("gpu/canary/nf4/%d" % K, N, K)
    p = w4.nf4_quantize(torch.from_numpy(W).to(DEV))
    xb = synth.to_bf16_bits(synth.activations("gpu/canary/nf4/x/%d" % M, M, K))
    obuf, ov = _guarded(2 * M * N)
    out = ov.view(torch.bfloat16).view(M, N)
    need = w4.nf4_workspace_bytes(M, N, K)
    wbuf, wv = _guarded(need)
    w4.nf4_gemm(bits_to_tensor(xb, "bf16"), p, out=out, workspace=wv if need > 0 else None)
    torch.cuda.synchronize()
    _check_guards(obuf, 2 * M * N, "output")
    _check_guards(wbuf, need, "workspace")
    codes, absmax = nf4.quantize_nf4(W, 64)
    aq, sc = nf4.double_quant(absmax)
    wd = nf4.dequant_nf4(nf4.pack_nf4(codes), aq, sc, 64, "bf16")
    assert compare_gemm(out, xb, wd, "bf16") <= TOL
