"""w4a16_gemm_noalloc, the entry point that allocates nothing (its workspace
is the library's fixed per-GPU scratch), against w4a16_gemm_bits with a
workspace of its own: the same kernels run, so the outputs are bitwise equal,
and both are within the oracle's tolerance.  Two calls in a row, the second
with a smaller input; the calls use the scratch (a permutation pass into it,
split-K partials in it)."""

import numpy as np
import pytest
import torch

import bit_weight_only_gemm_amd as w4
from bit_weight_only_gemm_amd import synth
from oracle import gemm
from gpu_util import DEV, say, bits_to_tensor, tensor_bits, int4_inputs, gpu_int4_pack, \
    oracle_int4_rows, compare_gemm

pytestmark = pytest.mark.gpu
TDT = {"f16": torch.float16, "bf16": torch.bfloat16}


def _one(tag, M, N, K, act, dtype):
    plan = w4.w4a16_gemm_plan(M, N, K, dtype=TDT[dtype], perm=act)
    say("noalloc", tag, M, N, K, act, dtype, plan)
    assert plan[0].startswith("w4a16::prep_") or plan[-1].startswith("w4a16::split_reduce_kernel")
    W, gi, _ = int4_inputs(tag, N, K, act_order=act)
    _, packed = gpu_int4_pack(W, gi)
    xb = synth.to_bits(synth.activations(tag + "/x", M, K), dtype)
    x = bits_to_tensor(xb, dtype)
    y_ws = w4.w4a16_gemm(x, packed)                     # a workspace of its own
    y_na = w4.w4a16_gemm_noalloc(x, packed)              # the fixed scratch
    torch.cuda.synchronize()
    assert np.array_equal(tensor_bits(y_na), tensor_bits(y_ws))
    wd = oracle_int4_rows(W, gi, np.arange(N), dtype)
    assert compare_gemm(y_na, xb, wd, dtype) <= gemm.TOL


def test_noalloc_equals_workspace_call_two_calls():
    # first call: the large-M kernel splitting K (fp32 partials in the scratch)
    # on a narrow layer; second, smaller: an act-order decode call whose
    # activations are permuted into the scratch first
    _one("gpu/noalloc/a", 64, 256, 4096, False, "bf16")
    _one("gpu/noalloc/b", 16, 512, 2048, True, "f16")


def test_noalloc_rejects_calls_beyond_the_scratch():
    # M * K * 2 bytes of permuted activations > 32 MiB: refused before launch
    M, N, K = 8192, 256, 4096
    assert w4.w4a16_workspace_bytes(M, N, K) > w4.NOALLOC_SCRATCH_BYTES
    W, gi, _ = int4_inputs("gpu/noalloc/big", N, K, act_order=True)
    _, packed = gpu_int4_pack(W, gi)
    x = torch.zeros((M, K), dtype=torch.float16, device=DEV)
    with pytest.raises(w4.W4A16Error, match="status 5"):
        w4.w4a16_gemm_noalloc(x, packed)
