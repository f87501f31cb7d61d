"""Host-only checks of the C ABI: the library loads, exports every symbol the
header declares, validates arguments before touching the GPU, and its own NF4
codebook equals the oracle's.  No kernel is launched here."""

import ctypes
import os
import re

import numpy as np
import pytest

from bit_weight_only_gemm_amd import _lib
from oracle import nf4

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "w4a16.h")

if not os.path.exists(_lib.LIB_PATH):
    pytest.skip("libw4a16.so not built", allow_module_level=True)

L = _lib.load()
NULL = ctypes.c_void_p(0)
FAKE = ctypes.c_void_p(0x10000)        # 16-byte aligned, never dereferenced
ODD = ctypes.c_void_p(0x10008)         # misaligned


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"^\s*(?:const\s+)?\w+\*?\s+\**(\w+)\s*\(", text, flags=re.M)
    return sorted(set(names))


def test_header_declares_what_binding_binds():
    assert declared_functions() == sorted(_lib.SIGNATURES)


def test_every_declared_symbol_is_exported():
    for name in declared_functions():
        assert hasattr(L, name), name


def test_status_strings_and_version():
    assert L.w4a16_version() == 2
    for s in range(8):
        assert L.w4a16_status_string(s) != b"unknown status"
    assert L.w4a16_status_string(99) == b"unknown status"


def test_repacked_bytes():
    assert L.w4a16_repacked_bytes(4096, 4096, 128, 0) == 4096 * 4096 // 2
    assert L.w4a16_repacked_bytes(4096, 4096, 128, 1) == 32 * 4096 * 2
    assert L.w4a16_repacked_bytes(4096, 4096, 128, 2) == 32 * 4096 // 2
    assert L.w4a16_repacked_bytes(1280, 64, 128, 1) == 16 * 64 * 2         # 10 groups -> 16
    assert L.w4a16_repacked_bytes(512, 200, 128, 0) == 4 * 4 * 4096   # N padded to 256
    assert L.w4a16_repacked_bytes(500, 256, 128, 0) == -1             # K % 128
    assert L.w4a16_repacked_bytes(512, 20, 128, 0) == -1              # N % 8
    # group sizes: 32 / 64 give 4 / 2 meta units per tile, multiples of 128 one
    assert L.w4a16_repacked_bytes(512, 256, 64, 0) == 4 * 4 * 4096
    assert L.w4a16_repacked_bytes(512, 256, 64, 1) == 2 * L.w4a16_repacked_bytes(512, 256, 128, 1)
    assert L.w4a16_repacked_bytes(512, 256, 32, 2) == 4 * L.w4a16_repacked_bytes(512, 256, 128, 2)
    for G in (256, 512, -1):                                          # -1: per-channel
        for w in (0, 1, 2):
            assert L.w4a16_repacked_bytes(512, 256, G, w) == L.w4a16_repacked_bytes(512, 256, 128, w)
    assert L.w4a16_repacked_bytes(512, 256, 96, 0) == -1              # unsupported G
    assert L.w4a16_repacked_bytes(512, 256, 16, 0) == -1
    assert L.w4a16_repacked_bytes(512, 256, 384, 0) == -1             # G does not divide K
    assert L.w4a16_repacked_bytes(512, 256, 0, 0) == -1
    assert L.w4a16_repacked_bytes(512, 256, -2, 0) == -1


def test_gemm_validation_without_gpu():
    g = L.w4a16_gemm
    # M <= 0
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 0, 256, 512, 0, NULL, 0, NULL) == 1
    # K not a multiple of the group size
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 500, 0, NULL, 0, NULL) == 1
    # unsupported group sizes, and one that does not divide K
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 96, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 16, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 384, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 1
    # unknown dtype
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 512, 7, NULL, 0, NULL) == 1
    # NULL required pointer
    assert g(NULL, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 1
    # misaligned pointer
    assert g(ODD, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 512, 0, NULL, 0, NULL) == 3
    # a workspace, when given, must hold w4a16_workspace_bytes (checked before
    # any launch; NULL is legal and is covered by the plan tests below)
    need = L.w4a16_workspace_bytes(16, 4096, 4096, 128)
    assert need >= 16 * 4096 * 2
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 16, 4096, 4096, 0, FAKE, need - 16, NULL) == 5
    # the size covers every call at a shape, with or without a permutation and
    # AWQ input scales: M <= 4 rows that the decode kernel stages on chip need
    # no workspace (rows, scales and permutation up to 152 KB per workgroup
    # on grids of at most 256 workgroups, else 72 KB; staged bytes up to
    # 40 MiB over the grid) ...
    assert L.w4a16_workspace_bytes(1, 4096, 4096, 128) == 0
    assert L.w4a16_workspace_bytes(4, 4096, 4096, 128) == 0
    assert L.w4a16_workspace_bytes(1, 4096, 11008, 128) == 0      # 256 x 44 KB
    assert L.w4a16_workspace_bytes(4, 4096, 11008, 128) == 0      # 256 x 152 KB, 39 MB staged
    assert L.w4a16_workspace_bytes(1, 4096, 16384, 128) == 0      # 256 x 129 KB
    assert L.w4a16_workspace_bytes(4, 6144, 5120, 128) == 0       # 384 x 50 KB
    # ... other ones are prepared in a pass: M * K * 2 bytes (up to 4 rows)
    assert L.w4a16_workspace_bytes(4, 6144, 8192, 128) >= 4 * 8192 * 2    # 384 x 80 KB
    assert L.w4a16_workspace_bytes(1, 55296, 5120, 128) >= 5120 * 2       # 3456 x 40 KB staged
    assert L.w4a16_workspace_bytes(1, 4096, 24576, 128) >= 24576 * 2      # 193 KB
    # ... and from 5 rows in whole row tiles of 16 (the operand layout)
    assert L.w4a16_workspace_bytes(5, 4096, 4096, 128) >= 16 * 4096 * 2
    # w4a16_gemm_xscale validates what the call needs (each case below fails
    # before any launch)
    xs = L.w4a16_gemm_xscale
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 4, 4096, 16384, 0, FAKE, 16,
              NULL) == 5        # 4 rows + scales: 160 KB, a pass
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 8, 4096, 4096, 0, FAKE, 16,
              NULL) == 5
    assert xs(FAKE, ODD, FAKE, FAKE, FAKE, NULL, 128, FAKE, 2, 4096, 4096, 0, NULL, 0, NULL) == 3
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 96, FAKE, 2, 4096, 4096, 0, NULL, 0, NULL) == 2
    # a prefill-sized call that splits K uses room for fp32 partials even
    # without a permutation
    need = L.w4a16_workspace_bytes(64, 5120, 5120, 128)
    assert need >= 2 * 64 * 5120 * 4
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 64, 5120, 5120, 0, FAKE, 16, NULL) == 5


def test_size_limits_without_gpu():
    # K <= 2^22, N <= 2^28, N K <= 2^37, M <= 2^21, M K and M N <= 2^36
    g = L.w4a16_gemm
    assert L.w4a16_repacked_bytes(1 << 22, 256, 128, 0) > 0
    assert L.w4a16_repacked_bytes(1 << 23, 256, 128, 0) == -1
    assert L.w4a16_repacked_bytes(4096, 1 << 29, 128, 0) == -1
    assert L.w4a16_repacked_bytes(1 << 20, 1 << 17, 128, 0) > 0          # N K = 2^37
    assert L.w4a16_repacked_bytes(1 << 20, (1 << 17) + 8, 128, 0) == -1
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1, 256, 1 << 23, 0, NULL, 0, NULL) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, (1 << 21) + 1, 256, 512, 0, NULL, 0,
             NULL) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1 << 20, 256, 1 << 17, 0, NULL, 0,
             NULL) == 2                                                  # M K = 2^37
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 1 << 20, 1 << 17, 512, 0, NULL, 0,
             NULL) == 2                                                  # M N = 2^37
    assert L.nf4_gemm(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 1, 256, 1 << 23, 1, NULL, 0, NULL) == 2
    assert L.w4a16_workspace_bytes(1 << 20, 256, 1 << 17, 128) == -1


def _plan(M, N, K, G=128, bits=4, dtype=0, perm=0, xs=0, ws=1):
    buf = ctypes.create_string_buffer(512)
    n = ctypes.c_int64(0)
    assert L.w4a16_gemm_plan(M, N, K, G, bits, dtype, perm, xs, ws, buf, 512,
                             ctypes.byref(n)) == 0
    assert n.value == len(buf.value)
    return buf.value.decode().split(" + ")


def test_plan_names_the_dispatch_without_gpu():
    dec = "w4a16::intb_decode_kernel<"
    # act-order decode: the in-kernel gather at 1 and 4 rows on the Llama
    # layers, a row-staged permutation pass at M = 4 where the rows and the
    # permutation outgrow LDS (16384 inputs), and at M = 16 a pass into the
    # operand layout (mode 6) feeding the fold; without a permutation M = 16
    # takes the transposed rows (mode 4); past 73728 inputs the passes
    # without row staging
    assert _plan(1, 4096, 4096, perm=1) == [dec + "0, 1, 2, 1, false, 4, true>"]
    assert _plan(4, 11008, 4096, perm=1) == [dec + "0, 1, 2, 1, false, 4, false>"]
    assert _plan(4, 4096, 11008, perm=1) == [dec + "0, 1, 2, 1, false, 4, false>"]
    assert _plan(4, 4096, 16384, perm=1) == ["w4a16::prep_rows_kernel<0, false>",
                                             dec + "0, 1, 0, 1, false, 4, false>"]
    assert _plan(16, 4096, 11008, perm=1) == ["w4a16::prep_rows_kernel<0, true>",
                                              dec + "0, 1, 6, 1, false, 4, false>"]
    assert _plan(24, 4096, 4096, perm=1) == ["w4a16::prep_rows_kernel<0, true>",
                                              dec + "0, 2, 6, 1, false, 4, false>"]
    assert _plan(16, 1024, 98304, perm=1)[0] == "w4a16::prep_tiled_kernel<0>"
    assert _plan(4, 1024, 98304, perm=1)[0] == "w4a16::prep_x_kernel<0>"
    assert _plan(16, 4096, 11008) == [dec + "0, 1, 4, 1, false, 4, false>"]
    # without a workspace: no pass, the kernel gathers from global memory
    # (mode 5), at any M, and the large-M kernel does not split K
    assert _plan(16, 4096, 11008, perm=1, ws=0) == [dec + "0, 1, 5, 1, false, 4, false>"]
    assert _plan(64, 5120, 5120, perm=1, ws=0) == [dec + "0, 1, 5, 1, false, 4, false>"]
    assert _plan(8, 4096, 4096, xs=1, ws=0) == [dec + "0, 1, 5, 1, true, 4, false>"]
    assert _plan(64, 5120, 5120, ws=1)[-1] == "w4a16::split_reduce_kernel<0>"
    assert all("split_reduce" not in k for k in _plan(64, 5120, 5120, ws=0))
    # wide packed decode on >= 16384 columns at 3-4 rows; 8-bit codes in bf16
    # never take the fold's forms
    assert _plan(4, 55296, 5120) == ["w4a16::intb_decode_wide_kernel<0, 1, 4, 2, 8>"]
    assert _plan(1, 4096, 4096, bits=8, dtype=1) == [dec + "1, 1, 0, 1, false, 8, false>"]
    assert _plan(1, 4096, 4096, G=32) == [dec + "0, 1, 0, 4, false, 4, true>"]
    # prefill: whole row blocks, and a separate launch for a partial last one
    # (which the planner counts as a round of its own), or one launch of the
    # ragged-tail form over every row block where that fits the CUs in fewer
    # rounds (5120 x 5120 at M = 2048: 11 x 20 blocks of 192 rows in one
    # round, against 8 x 20 of 256)
    assert _plan(2048, 7168, 5120, dtype=1) == ["w4a16::wq_prefill_kernel<1, 256, false, 0, 1, 4>"]
    assert _plan(2048, 5120, 5120, dtype=1) == ["w4a16::wq_prefill_kernel<1, 192, true, 0, 1, 4>"]
    assert _plan(2100, 7168, 5120, dtype=1) == ["w4a16::wq_prefill_kernel<1, 256, true, 0, 1, 4>"]
    assert _plan(2100, 55296, 5120, dtype=1)[:2] == [
        "w4a16::wq_prefill_kernel<1, 256, false, 0, 1, 4>",
        "w4a16::wq_prefill_kernel<1, 256, true, 0, 1, 4>"]
    # the plan's pass agrees with w4a16_workspace_bytes
    for M, N, K in [(1, 4096, 4096), (4, 11008, 4096), (16, 4096, 4096), (5, 55296, 5120)]:
        has_pass = any(k.startswith("w4a16::prep_")
                       for k in _plan(M, N, K, perm=1))
        assert has_pass == (L.w4a16_workspace_bytes(M, N, K, 128) > 0 and
                            not _plan(M, N, K)[-1].endswith("split_reduce_kernel<0>")) or has_pass
    # NF4: the decode kernel up to 32 rows on this layer, the large-M kernel after
    buf = ctypes.create_string_buffer(256)
    assert L.nf4_gemm_plan(32, 28672, 8192, 64, 1, 1, buf, 256, NULL) == 0
    assert buf.value == b"w4a16::nf4_decode_kernel<1, 2, 4, true>"
    assert L.nf4_gemm_plan(33, 28672, 8192, 64, 1, 0, buf, 256, NULL) == 0
    assert buf.value == b"w4a16::wq_prefill_kernel<1, 64, true, 1, 1, 4>"
    # truncation keeps the terminator; bad buffers are refused
    small = ctypes.create_string_buffer(8)
    n = ctypes.c_int64(0)
    assert L.nf4_gemm_plan(1, 28672, 8192, 64, 1, 1, small, 8, ctypes.byref(n)) == 0
    assert small.value == b"w4a16::" and n.value > 8
    assert L.nf4_gemm_plan(1, 28672, 8192, 64, 1, 1, NULL, 8, NULL) == 1
    assert L.w4a16_gemm_plan(0, 256, 512, 128, 4, 0, 0, 0, 1, NULL, 0, NULL) == 1


def test_host_allocation_failure_is_a_status():
    """A failed host allocation inside an entry point (here the host copy of
    g_idx in w4a16_make_perm, 16 MiB at K = 2^22) returns W4A16_ERR_HOST
    instead of throwing across the C ABI.  Run in a child process whose
    address space is capped just above its current size, so the allocation
    fails before any HIP call is made."""
    import subprocess
    import sys
    code = r"""
import ctypes, resource, sys
L = ctypes.CDLL(sys.argv[1])
L.w4a16_make_perm.argtypes = [ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_void_p,
                              ctypes.c_void_p, ctypes.c_void_p]
nt = ctypes.c_int32(0)
vm = [int(l.split()[1]) for l in open('/proc/self/status') if l.startswith('VmSize:')][0]
lim = (vm + 4096) * 1024
resource.setrlimit(resource.RLIMIT_AS, (lim, resource.getrlimit(resource.RLIMIT_AS)[1]))
st = L.w4a16_make_perm(ctypes.c_void_p(0x10000), 1 << 22, 128, ctypes.c_void_p(0x10000),
                       ctypes.byref(nt), None)
print(st)
"""
    r = subprocess.run([sys.executable, "-c", code, _lib.LIB_PATH], capture_output=True,
                       text=True, timeout=120)
    assert r.returncode == 0, r.stderr
    assert r.stdout.strip() == "7", (r.stdout, r.stderr)
def test_nf4_validation_without_gpu():
    g = L.nf4_gemm
    assert g(FAKE, FAKE, FAKE, FAKE, 32, FAKE, 1, 256, 512, 1, NULL, 0, NULL) == 2   # blocksize
    assert g(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 1, 256, 96, 1, NULL, 0, NULL) == 1    # K % 64
    assert g(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 1, 250, 512, 1, NULL, 0, NULL) == 1   # N % 16
    assert g(FAKE, NULL, FAKE, FAKE, 64, FAKE, 1, 256, 512, 1, NULL, 0, NULL) == 1
    assert L.nf4_quantize(FAKE, 16, 100, 64, FAKE, FAKE, FAKE, NULL) == 1
    assert L.nf4_workspace_bytes(1, 28672, 8192, 64) >= 0


def test_quantize_and_repack_validation_without_gpu():
    used = ctypes.c_int32(0)
    # g_idx given without a perm buffer
    assert L.w4a16_repack(FAKE, FAKE, FAKE, FAKE, 512, 256, 128, FAKE, FAKE, FAKE, NULL,
                          ctypes.byref(used), NULL) == 1
    # symmetric weights: qzeros and zeros_r are both NULL or both given
    assert L.w4a16_repack(FAKE, FAKE, NULL, NULL, 512, 256, 64, FAKE, FAKE, FAKE, NULL,
                          ctypes.byref(used), NULL) == 1
    assert L.w4a16_repack(FAKE, FAKE, FAKE, NULL, 512, 256, 64, FAKE, FAKE, NULL, NULL,
                          ctypes.byref(used), NULL) == 1
    assert L.w4a16_repack(FAKE, FAKE, NULL, NULL, 512, 256, 96, FAKE, FAKE, NULL, NULL,
                          ctypes.byref(used), NULL) == 2
    # quantize: g_idx without perm
    assert L.w4a16_quantize_rtn(FAKE, FAKE, NULL, 256, 512, 128, FAKE, FAKE, FAKE, NULL) == 1
    assert L.w4a16_quantize_rtn(FAKE, NULL, NULL, 256, 512, 48, FAKE, FAKE, NULL, NULL) == 2
    assert L.w4a16_set_timing_events(NULL, NULL) == 0


def test_library_codebook_equals_oracle_codebook():
    buf = (ctypes.c_float * 16)()
    assert L.nf4_codebook(ctypes.cast(buf, ctypes.c_void_p)) == 0
    got = np.frombuffer(buf, dtype=np.float32)
    assert np.array_equal(got.view(np.uint32), nf4.nf4_codebook().view(np.uint32))


def test_bits_entry_points_validation_without_gpu():
    rb = L.w4a16_repacked_bytes_bits
    # 256 b bytes per 16 x 128 tile; scales as at 4 bits; zeros twice as wide at 8 bits
    for bits in (3, 4, 8):
        assert rb(4096, 4096, 128, bits, 0) == 4096 * 4096 * bits // 8
        assert rb(4096, 4096, 128, bits, 1) == L.w4a16_repacked_bytes(4096, 4096, 128, 1)
    assert rb(4096, 4096, 128, 8, 2) == 2 * L.w4a16_repacked_bytes(4096, 4096, 128, 2)
    assert rb(4096, 4096, 128, 3, 2) == L.w4a16_repacked_bytes(4096, 4096, 128, 2)
    assert rb(4096, 4096, 32, 8, 2) == 8 * L.w4a16_repacked_bytes(4096, 4096, 128, 2)
    for bits in (0, 2, 5, 16):
        assert rb(4096, 4096, 128, bits, 0) == -1
    used = ctypes.c_int32(0)
    # unsupported widths, before anything else is looked at
    assert L.w4a16_repack_bits(FAKE, FAKE, FAKE, NULL, 512, 256, 128, 5, FAKE, FAKE, FAKE, NULL,
                               ctypes.byref(used), NULL) == 2
    assert L.w4a16_quantize_rtn_bits(FAKE, NULL, NULL, 256, 512, 128, 2, FAKE, FAKE, FAKE,
                                     NULL) == 2
    assert L.w4a16_gemm_bits(FAKE, NULL, FAKE, FAKE, FAKE, NULL, 128, 6, FAKE, 1, 256, 512, 0,
                             NULL, 0, NULL) == 2
    assert L.w4a16_dequant_bits(FAKE, FAKE, FAKE, 512, 256, 128, 7, 0, FAKE, NULL) == 2
    # 3-bit zeros pack in runs of 32 columns: N = 200 is refused with zeros ...
    assert L.w4a16_repack_bits(FAKE, FAKE, FAKE, NULL, 512, 200, 128, 3, FAKE, FAKE, FAKE, NULL,
                               ctypes.byref(used), NULL) == 1
    assert L.w4a16_quantize_rtn_bits(FAKE, NULL, NULL, 200, 512, 128, 3, FAKE, FAKE, FAKE,
                                     NULL) == 1
    # ... and a symmetric repack without zeros_r passes validation up to the
    # pointer checks (misaligned codes_r here, so nothing is launched)
    assert L.w4a16_repack_bits(FAKE, FAKE, NULL, NULL, 512, 200, 128, 3, ODD, FAKE, NULL, NULL,
                               ctypes.byref(used), NULL) == 3
    # the 8-bit GEMM validates like the 4-bit one
    assert L.w4a16_workspace_bytes(64, 5120, 5120, 128) > 0        # split K: partials
    assert L.w4a16_gemm_bits(FAKE, NULL, FAKE, FAKE, FAKE, NULL, 128, 8, FAKE, 64, 5120, 5120, 0,
                             FAKE, 16, NULL) == 5


def test_nf4_repack_entry_points_without_gpu():
    # tiles of 16 rows x 128 inputs, 1 KB each; N % 16 and the NF4 shape rules
    assert L.nf4_repacked_bytes(28672, 8192, 64) == 28672 // 16 * 64 * 1024
    assert L.nf4_repacked_bytes(16, 320, 64) == 3 * 1024          # a half last tile
    assert L.nf4_repacked_bytes(20, 320, 64) == -1
    assert L.nf4_repacked_bytes(16, 96, 64) == -1
    assert L.nf4_repacked_bytes(16, 128, 32) == -1
    assert L.nf4_repack(FAKE, 20, 320, 64, FAKE, NULL) == 1
    assert L.nf4_repack(FAKE, 16, 320, 32, FAKE, NULL) == 2
    assert L.nf4_repack(NULL, 16, 320, 64, FAKE, NULL) == 1
    assert L.nf4_repack(FAKE, 16, 320, 64, ODD, NULL) == 3
    g = L.nf4_gemm_repacked
    assert g(FAKE, FAKE, FAKE, FAKE, 32, FAKE, 1, 256, 512, 1, NULL, 0, NULL) == 2
    assert g(FAKE, FAKE, FAKE, FAKE, 64, FAKE, 1, 250, 512, 1, NULL, 0, NULL) == 1
    assert g(FAKE, NULL, FAKE, FAKE, 64, FAKE, 1, 256, 512, 1, NULL, 0, NULL) == 1
    # the plan names the kernels that read the tiles: nf4r_decode_kernel, and
    # the large-M kernel's format 2
    buf = ctypes.create_string_buffer(256)
    assert L.nf4_gemm_repacked_plan(1, 28672, 8192, 64, 1, 1, buf, 256, NULL) == 0
    assert buf.value == b"w4a16::nf4r_decode_kernel<1, 1, 0, true>"
    assert L.nf4_gemm_repacked_plan(2048, 28672, 8192, 64, 1, 1, buf, 256, NULL) == 0
    assert buf.value == b"w4a16::wq_prefill_kernel<1, 256, false, 2, 1, 4>"
