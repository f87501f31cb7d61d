"""The preparation passes of calls with a workspace: x_p[m, k] =
x[m, perm[k]] / s[perm[k]] written once per call, then read by the GEMM.

Forms (the plan query names each call's kernels in the test output):
prep_rows_kernel (each row staged in LDS by DMA, the permutation in
registers) in row-major form (packed decode at up to 4 rows, the large-M
kernel) and in the decode kernel's operand layout (TILED, more than 4 rows,
one and two row tiles); and, past what LDS holds (K > 73728, or K > 36864
with input scales), prep_x_kernel and prep_tiled_kernel.  Every output is
compared with the oracle (act-order weights in their original column order,
[P2] §三 3.1 `desc_act`; AWQ input scales, [P3] §4.1) within the tolerance.
"""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import gemm
from gpu_util import say, bits_to_tensor, tensor_f64, int4_inputs, gpu_int4_pack, oracle_int4_rows

pytestmark = pytest.mark.gpu
TOL = gemm.TOL
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}

# (M, N, K, act-order, input scales, dtype, the pass the plan must name)
CASES = [
    (4, 256, 16384, True, False, "f16", "prep_rows_kernel<0, false>"),
    (3, 208, 16384, True, True, "bf16", "prep_rows_kernel<1, false>"),
    (16, 208, 11008, True, False, "bf16", "prep_rows_kernel<1, true>"),
    (13, 256, 4096, False, True, "f16", "prep_rows_kernel<0, true>"),
    (20, 208, 4096, True, True, "f16", "prep_rows_kernel<0, true>"),
    (64, 256, 2048, True, False, "bf16", "prep_rows_kernel<1, false>"),
    (5, 208, 77824, True, False, "f16", "prep_tiled_kernel<0>"),
    (4, 208, 77824, True, False, "bf16", "prep_x_kernel<1>"),
    (8, 208, 40960, False, True, "f16", "prep_tiled_kernel<0>"),
]


@pytest.mark.parametrize("M,N,K,act,xs,dtype,pass_name", CASES)
def test_prepared_activations_match_oracle(M, N, K, act, xs, dtype, pass_name):
    tag = "gpu/prep/%d/%d/%d/%d" % (M, K, act, xs)
    plan = w4.w4a16_gemm_plan(M, N, K, dtype=TDT[dtype], perm=act, x_scale=xs)
    say("prep", M, N, K, act, xs, dtype, plan)
    assert plan[0] == "w4a16::" + pass_name
    W, gi, s = int4_inputs(tag, N, K, act_order=act, awq=xs)
    _, packed = gpu_int4_pack(W, gi)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    if xs:
        sb = synth.to_bits(s[None, :], dtype)[0]
        y = w4.w4a16_gemm_xscale(bits_to_tensor(xb, dtype), bits_to_tensor(sb, dtype), packed)
        torch.cuda.synchronize()
        err = gemm.rel_err(tensor_f64(y, dtype), gemm.gemm_ref_xscale_bits(xb, sb, wd, dtype))
    else:
        y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
        torch.cuda.synchronize()
        err = gemm.rel_err(tensor_f64(y, dtype), gemm.gemm_ref_bits(xb, wd, dtype))
    say("  rel err", err)
    assert err <= TOL


# (M, K, input scales, dtype): 1-4 rows gathered and scaled on chip by the
# decode kernel itself, the rows and the permutation staged in LDS and each
# operand gathered in the loop (one row: a quad's lanes gather 2 inputs each
# and share them), up to what LDS holds (4 rows of 12288 inputs with the
# permutation; 4 rows of 11008 with the permutation and input scales)
STAGED = [(1, 11008, False, "f16"), (2, 11008, True, "bf16"), (3, 11008, False, "bf16"),
          (4, 11008, True, "f16"), (4, 12288, False, "f16"), (3, 4096, True, "f16"),
          (1, 16384, False, "bf16"), (1, 4096, True, "bf16"), (2, 16384, False, "f16")]


@pytest.mark.parametrize("M,K,xs,dtype", STAGED)
def test_staged_gather_matches_oracle(M, K, xs, dtype):
    N = 208
    tag = "gpu/prep/staged/%d/%d/%d" % (M, K, xs)
    plan = w4.w4a16_gemm_plan(M, N, K, dtype=TDT[dtype], perm=True, x_scale=xs)
    say("staged gather", M, N, K, xs, dtype, plan)
    assert plan == ["w4a16::intb_decode_kernel<%d, 1, 2, 1, %s, 4, %s>"
                    % (0 if dtype == "f16" else 1, "true" if xs else "false",
                       "true" if M == 1 else "false")]
    W, gi, s = int4_inputs(tag, N, K, act_order=True, awq=xs)
    _, packed = gpu_int4_pack(W, gi)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    if xs:
        sb = synth.to_bits(s[None, :], dtype)[0]
        y = w4.w4a16_gemm_xscale(bits_to_tensor(xb, dtype), bits_to_tensor(sb, dtype), packed)
        torch.cuda.synchronize()
        err = gemm.rel_err(tensor_f64(y, dtype), gemm.gemm_ref_xscale_bits(xb, sb, wd, dtype))
    else:
        y = w4.w4a16_gemm(bits_to_tensor(xb, dtype), packed)
        torch.cuda.synchronize()
        err = gemm.rel_err(tensor_f64(y, dtype), gemm.gemm_ref_bits(xb, wd, dtype))
    say("  rel err", err)
    assert err <= TOL
