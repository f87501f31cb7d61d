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
    assert L.w4a16_version() == 1
    for s in range(7):
        assert L.w4a16_status_string(s)
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
    # a permutation needs a workspace of w4a16_workspace_bytes
    need = L.w4a16_workspace_bytes(16, 4096, 4096, 128)
    assert need >= 16 * 4096 * 2
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 16, 4096, 4096, 0, FAKE, need - 16, NULL) == 5
    assert g(FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 16, 4096, 4096, 0, NULL, 0, NULL) == 5
    # the size covers every call at a shape, with or without a permutation and
    # AWQ input scales: M <= 4 rows (with the permutation and the scales) that
    # the decode kernel stages on chip need no workspace (up to 72 KB per
    # workgroup and 17 MiB over the grid: 256 x 24 KB and 256 x 56 KB here) ...
    assert L.w4a16_workspace_bytes(1, 4096, 4096, 128) == 0
    assert L.w4a16_workspace_bytes(4, 4096, 4096, 128) == 0
    # ... larger ones are prepared in a pass: M * K * 2 bytes
    assert L.w4a16_workspace_bytes(1, 4096, 11008, 128) >= 11008 * 2     # 88 KB per workgroup
    assert L.w4a16_workspace_bytes(4, 6144, 4096, 128) >= 4 * 4096 * 2    # 384 x 56 KB
    assert L.w4a16_workspace_bytes(1, 55296, 5120, 128) >= 5120 * 2        # 3456 workgroups
    assert L.w4a16_workspace_bytes(4, 4096, 11008, 128) >= 4 * 11008 * 2
    assert L.w4a16_workspace_bytes(5, 4096, 4096, 128) >= 5 * 4096 * 2
    # w4a16_gemm_xscale validates what the call needs (each case below fails
    # before any launch)
    xs = L.w4a16_gemm_xscale
    # scales with rows that do not fit on chip, and with M > 4: a pass
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 4, 4096, 11008, 0, NULL, 0, NULL) == 5
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, FAKE, 128, FAKE, 4, 4096, 11008, 0, NULL, 0, NULL) == 5
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 8, 4096, 4096, 0, NULL, 0, NULL) == 5
    assert xs(FAKE, ODD, FAKE, FAKE, FAKE, NULL, 128, FAKE, 2, 4096, 4096, 0, NULL, 0, NULL) == 3
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 96, FAKE, 2, 4096, 4096, 0, NULL, 0, NULL) == 2
    assert xs(FAKE, FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 64, 5120, 5120, 0, NULL, 0,
              NULL) == 5
    # a prefill-sized call that splits K needs room for fp32 partials even
    # without a permutation
    need = L.w4a16_workspace_bytes(64, 5120, 5120, 128)
    assert need >= 2 * 64 * 5120 * 4
    assert g(FAKE, FAKE, FAKE, FAKE, NULL, 128, FAKE, 64, 5120, 5120, 0, NULL, 0, NULL) == 5


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
                             NULL, 0, NULL) == 5
