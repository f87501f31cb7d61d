"""Pins for oracle/int4.py: brute force, closed forms, exhaustive dequant, invariances."""

import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import int4, gemm
from bit_weight_only_gemm_amd import synth


# ---------------------------------------------------------------- packing (P1)

def test_qweight_pack_unpack_exhaustive_positions():
    # every (position, value) pair in a word, including top nibbles >= 8
    K, N = 8, 1
    for j in range(8):
        for v in range(16):
            q = np.zeros((N, K), dtype=np.uint8)
            q[0, j] = v
            w = int4.pack_qweight(q)
            assert w.dtype == np.int32 and w.shape == (1, 1)
            assert int(w.view(np.uint32)[0, 0]) == v << (4 * j)
            assert np.array_equal(int4.unpack_qweight(w), q)


def test_qweight_roundtrip_random_words():
    r = np.random.default_rng(3)
    words = r.integers(0, 2**32, size=(64, 256), dtype=np.uint64).astype(np.uint32).view(np.int32)
    assert (words < 0).any()
    q = int4.unpack_qweight(words)
    assert q.shape == (256, 512) and q.max() <= 15
    assert np.array_equal(int4.pack_qweight(q), words)


def test_qzeros_pack_unpack():
    r = np.random.default_rng(4)
    z = r.integers(0, 16, size=(5, 64)).astype(np.uint8)
    w = int4.pack_qzeros(z)
    assert w.shape == (5, 8)
    assert np.array_equal(int4.unpack_qzeros(w), z)
    # nibble j of word i is the zero of column 8i + j
    assert int(w.view(np.uint32)[2, 3]) & 0xF == z[2, 24]
    assert (int(w.view(np.uint32)[2, 3]) >> 28) & 0xF == z[2, 31]


# ------------------------------------------------------------ quantizer (P2, P3)

def test_rtn_hand_example():
    # One group of 8 values, worked by hand:
    #   min = -0.3, max = 0.45 -> (max - min) / 15 = 0.05 (fp32) -> fp16 scale
    #   s = 1638 / 1024 * 2^-5 = 0.0499877929...  (0.05 * 2^5 * 1024 = 1638.4)
    #   z = rint(0.3 / s) = rint(6.0015) = 6
    #   w / s = [-6.0015, -2.0005, 0, 1.0002, 3.0007, 4.0010, 7.0017, 9.0022]
    #   q = rint(w / s) + 6 = [0, 4, 6, 7, 9, 10, 13, 15]
    w = np.array([[-0.3, -0.1, 0.0, 0.05, 0.15, 0.2, 0.35, 0.45]], dtype=np.float32)
    q, s, z = int4.quantize_rtn_int4(w, group_size=8)
    assert float(s[0, 0]) == 1638 / 1024 * 2.0**-5
    assert int(z[0, 0]) == 6
    assert q[0].tolist() == [0, 4, 6, 7, 9, 10, 13, 15]


def test_rtn_codes_in_range_and_roundtrip_bound():
    W = synth.weights("test/rtn/W", 64, 1024)
    q, s, z = int4.quantize_rtn_int4(W, 128)
    assert q.max() <= 15 and z.max() <= 15
    sf = s.astype(np.float64)[np.arange(1024) // 128].T          # [N, K]
    zf = z.astype(np.float64)[np.arange(1024) // 128].T
    deq = (q.astype(np.float64) - zf) * sf
    err = np.abs(W.astype(np.float64) - deq) / sf
    clamped = (q == 0) | (q == 15)
    # unclamped codes are the nearest level: |w - deq| <= s/2 (fp32 division slack)
    assert err[~clamped].max() <= 0.5 + 1e-6
    # clamped codes: s is an fp16 round of range/15, so the bound is s*(1/2 + 15*2^-11)
    assert err[clamped].max() <= 0.5 + 15 * 2.0**-11 + 1e-6


def test_rtn_is_nearest_level_brute_force():
    # for each weight, no other code in [0, 15] is strictly closer (given s, z)
    W = synth.weights("test/rtn/brute", 4, 256)
    q, s, z = int4.quantize_rtn_int4(W, 128)
    g = np.arange(256) // 128
    for n in range(4):
        for k in range(0, 256, 7):
            sf = np.float64(s[g[k], n])
            levels = (np.arange(16) - np.float64(z[g[k], n])) * sf
            d = np.abs(levels - np.float64(W[n, k]))
            assert d[q[n, k]] <= d.min() + 1e-6 * sf


def test_rtn_degenerate_group():
    W = np.full((2, 128), 0.3, dtype=np.float32)
    W[1] = -7.25
    q, s, z = int4.quantize_rtn_int4(W, 128)
    assert float(s[0, 0]) == 1.0 and float(s[0, 1]) == 1.0
    deq = (q.astype(np.int64) - z[0][:, None].astype(np.int64)) * 1.0
    assert np.abs(deq - W.astype(np.float64)).max() <= 0.5


# ---------------------------------------------------------- dequant (P4, exhaustive)

def _f16_of_exact(v):
    if abs(v) >= 65520.0:
        return np.float16(np.inf if v > 0 else -np.inf).view(np.uint16)
    return np.uint16(struct.unpack("<H", struct.pack("<e", v))[0])


def _scale_set():
    r = np.random.default_rng(5)
    pows = [2.0**e for e in range(-14, 12)]
    rand = list(r.standard_normal(24).astype(np.float16).astype(float))
    sub = [2.0**-24, 3 * 2.0**-24, 1023 * 2.0**-24, 2.0**-20 + 2.0**-24]
    big = [4096.0, 4368.0, 60000.0, 65504.0]
    vals = pows + rand + sub + big + [0.0, -0.0]
    return np.array(vals, dtype=np.float16)


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dequant_exhaustive_vs_exact_rational(dtype):
    scales = _scale_set()
    N = 16
    K = 16 * len(scales) * 8                   # one group of 8 per (q-row, scale)
    # build canonical tensors with group size 8: rows n = z, columns cycle q
    G = 8
    ng = K // G
    q = np.tile(np.arange(16, dtype=np.uint8), (N, K // 16))            # [N, K]
    z = np.tile(np.arange(N, dtype=np.uint8)[None, :], (ng, 1))         # [ng, N]
    s = np.repeat(scales, ng // len(scales) + 1)[:ng]
    s = np.tile(s[:, None], (1, N)).astype(np.float16)
    got = int4.dequant_int4(int4.pack_qweight(q), s, int4.pack_qzeros(z), None, G, dtype)
    for n in range(N):
        for k in range(0, K, 3):
            g = k // G
            exact = Fraction(int(q[n, k]) - int(z[g, n])) * Fraction(float(s[g, n]))
            if dtype == "f16":
                want = _f16_of_exact(float(exact))
            else:
                t = torch.tensor([float(exact)], dtype=torch.float64).to(torch.bfloat16)
                want = t.view(torch.int16).numpy().view(np.uint16)[0]
            gv, wv = int(got[n, k]), int(want)
            if (gv & 0x7FFF) == 0 and (wv & 0x7FFF) == 0:
                # a zero product: sign is that of (q - z) * s under IEEE rules
                sign = np.signbit(np.float32(int(q[n, k]) - int(z[g, n])) * np.float32(s[g, n]))
                assert (gv >> 15) == int(sign)
                continue
            assert gv == wv, (n, k, int(q[n, k]), int(z[g, n]), float(s[g, n]), dtype)


def test_dequant_gather_form_with_g_idx():
    K, N, G = 512, 32, 128
    W = synth.weights("test/deq/gidx", N, K)
    gi = synth.act_order_gidx("test/deq/gidx/g", K, G)
    q, s, z = int4.quantize_rtn_int4(W, G, gi)
    wd = int4.dequant_int4(int4.pack_qweight(q), s, int4.pack_qzeros(z), gi, G, "f16")
    # independent per-element formula
    for n in range(0, N, 5):
        for k in range(0, K, 11):
            g = gi[k]
            v = np.float32(np.float32(int(q[n, k]) - int(z[g, n])) * np.float32(s[g, n]))
            assert wd[n, k] == v.astype(np.float16).view(np.uint16)


# ------------------------------------------------------------ g_idx invariance (P5)

def test_trivial_gidx_equals_none():
    K, N, G = 384, 16, 128
    W = synth.weights("test/gidx/trivial", N, K)
    a = int4.quantize_rtn_int4(W, G, None)
    b = int4.quantize_rtn_int4(W, G, int4.default_g_idx(K, G))
    for u, v in zip(a, b):
        assert np.array_equal(u, v)


def test_act_order_equals_contiguous_groups_of_permuted_columns():
    K, N, G = 512, 24, 128
    W = synth.weights("test/gidx/perm/W", N, K)
    gi = synth.act_order_gidx("test/gidx/perm/g", K, G)
    perm = np.argsort(gi, kind="stable")
    q1, s1, z1 = int4.quantize_rtn_int4(W, G, gi)
    q2, s2, z2 = int4.quantize_rtn_int4(W[:, perm], G, None)
    assert np.array_equal(q1[:, perm], q2)
    assert np.array_equal(s1, s2) and np.array_equal(z1, z2)
    d1 = int4.dequant_int4(int4.pack_qweight(q1), s1, int4.pack_qzeros(z1), gi, G, "f16")
    d2 = int4.dequant_int4(int4.pack_qweight(q2), s2, int4.pack_qzeros(z2), None, G, "f16")
    assert np.array_equal(d1[:, perm], d2)
    x = synth.to_f16_bits(synth.activations("test/gidx/perm/x", 3, K))
    y1 = gemm.gemm_ref_bits(x, d1, "f16")
    y2 = gemm.gemm_ref_bits(x, d2, "f16", perm=perm)
    assert gemm.rel_err(y1, y2) < 1e-13


def test_q_equal_z_gives_zero_product():
    K, N, G = 256, 8, 128
    z = np.random.default_rng(6).integers(0, 16, size=(K // G, N)).astype(np.uint8)
    q = z[np.arange(K) // G].T.copy()
    s = np.full((K // G, N), 0.01, dtype=np.float16)
    wd = int4.dequant_int4(int4.pack_qweight(q), s, int4.pack_qzeros(z), None, G, "f16")
    assert not np.any(wd & 0x7FFF)


# ------------------------------------------- group sizes and symmetric codes (P2, P3)

def _fp16_scales(r, shape):
    # fp16 values with at most 11 significant bits: 15 s and 7 s are exact in fp32
    return (r.uniform(0.002, 0.05, size=shape).astype(np.float16)).astype(np.float32)


@pytest.mark.parametrize("G", [32, 64, 128, 256, 1024])
def test_rtn_recovers_an_exact_grid_per_group(G):
    # w = (q - z) s with every (row, group) holding codes 0 and 15: then
    # (max - min) / 15 = s, rint(-min / s) = z and rint(w / s) + z = q exactly,
    # so a wrong group boundary (a different s or z) cannot reproduce q, s, z
    N, K = 6, 1024
    r = np.random.default_rng(21 + G)
    ng = K // G
    s = _fp16_scales(r, (ng, N))
    z = r.integers(0, 16, size=(ng, N))
    q = r.integers(0, 16, size=(N, K))
    for g in range(ng):
        q[:, g * G] = 0
        q[:, g * G + G - 1] = 15
    gk = np.arange(K) // G
    W = ((q - z[gk].T) * s[gk].T).astype(np.float32)
    q2, s2, z2 = int4.quantize_rtn_int4(W, G)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    assert np.array_equal(s2.astype(np.float32), s)


@pytest.mark.parametrize("G", [32, 64, 128, 1024])
def test_symmetric_rtn_recovers_an_exact_grid(G):
    # w = c s, c in [-7, 7] with |c| = 7 in every (row, group): max|w| / 7 = s
    # and rint(w / s) = c exactly; the stored nibble is c + 8, no zeros
    N, K = 5, 1024
    r = np.random.default_rng(40 + G)
    ng = K // G
    s = _fp16_scales(r, (ng, N))
    c = r.integers(-7, 8, size=(N, K))
    for g in range(ng):
        c[:, g * G + 3] = np.where(r.random(N) < 0.5, 7, -7)
    gk = np.arange(K) // G
    W = (c * s[gk].T).astype(np.float32)
    q, s2, z = int4.quantize_rtn_int4(W, G, sym=True)
    assert z is None
    assert np.array_equal(q.astype(np.int64), c + 8)
    assert np.array_equal(s2.astype(np.float32), s)


def test_symmetric_rtn_is_odd():
    # rint is symmetric and max|w| is sign-blind: negating W mirrors every code
    # about the zero nibble 8 (codes stay in [1, 15]: -8 is never produced)
    W = synth.weights("test/sym/odd", 16, 512)
    q1, s1, _ = int4.quantize_rtn_int4(W, 64, sym=True)
    q2, s2, _ = int4.quantize_rtn_int4(-W, 64, sym=True)
    assert q1.min() >= 1 and q2.min() >= 1
    assert np.array_equal(q2.astype(np.int64), 16 - q1.astype(np.int64))
    assert np.array_equal(s1, s2)


@pytest.mark.parametrize("G", [32, 64])
def test_symmetric_rtn_nearest_level_brute_force(G):
    W = synth.weights(f"test/sym/brute/{G}", 4, 256)
    q, s, _ = int4.quantize_rtn_int4(W, G, sym=True)
    for n in range(4):
        for k in range(0, 256, 5):
            sf = np.float64(s[k // G, n])
            levels = np.arange(-8, 8) * sf                 # nibbles 0..15
            d = np.abs(levels - np.float64(W[n, k]))
            assert d[q[n, k]] <= d.min() + 1e-6 * sf
            # and the error bound of a rounding to a grid of step s
            assert d[q[n, k]] <= 0.5 * sf * (1 + 1e-6)


def test_symmetric_degenerate_and_zero_group():
    W = np.zeros((2, 64), dtype=np.float32)
    W[1, 5] = 3.5
    q, s, _ = int4.quantize_rtn_int4(W, 32, sym=True)
    assert float(s[0, 0]) == 1.0 and np.all(q[0] == 8)       # all-zero group: s = 1
    assert float(s[0, 1]) == 0.5 and q[1, 5] == 15 and q[1, 4] == 8
    assert float(s[1, 1]) == 1.0


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_symmetric_dequant_exact_and_mirrored(dtype):
    # no zeros: w = (q - 8) s exactly rounded; nibble 8 is +0 and nibbles
    # 8 + k and 8 - k give values of opposite sign and equal magnitude
    scales = _scale_set()
    scales = scales[np.isfinite(scales.astype(np.float32)) & (scales != 0)]
    G = 16
    K = G * len(scales)
    q = np.tile(np.arange(16, dtype=np.uint8), (3, K // 16))
    s = np.tile(scales[:, None], (1, 3)).astype(np.float16)
    got = int4.dequant_int4(int4.pack_qweight(q), s, None, None, G, dtype)
    for k in range(K):
        sv = Fraction(float(scales[k // G]))
        exact = Fraction(int(q[0, k]) - 8) * sv
        if dtype == "f16":
            want = int(_f16_of_exact(float(exact)))
        else:
            t = torch.tensor([float(exact)], dtype=torch.float64).to(torch.bfloat16)
            want = int(t.view(torch.int16).numpy().view(np.uint16)[0])
        if q[0, k] == 8:
            want = 0 if float(scales[k // G]) > 0 else 0x8000
        assert int(got[0, k]) == want, (k, int(q[0, k]), float(scales[k // G]))
    for k0 in range(0, K, 16):
        for d in range(1, 8):
            a, b = int(got[0, k0 + 8 + d]), int(got[0, k0 + 8 - d])
            assert a ^ b == 0x8000


def test_symmetric_equals_asymmetric_with_zero_eight():
    K, N, G = 256, 16, 64
    W = synth.weights("test/sym/z8", N, K)
    q, s, _ = int4.quantize_rtn_int4(W, G, sym=True)
    z8 = np.full((K // G, N), 8, dtype=np.uint8)
    a = int4.dequant_int4(int4.pack_qweight(q), s, None, None, G, "bf16")
    b = int4.dequant_int4(int4.pack_qweight(q), s, int4.pack_qzeros(z8), None, G, "bf16")
    assert np.array_equal(a, b)


@pytest.mark.parametrize("sym", [False, True])
def test_small_group_act_order_equals_contiguous_groups(sym):
    K, N, G = 512, 16, 32
    W = synth.weights(f"test/gidx/g32/{sym}", N, K)
    gi = synth.act_order_gidx(f"test/gidx/g32/g/{sym}", K, G)
    perm = np.argsort(gi, kind="stable")
    q1, s1, z1 = int4.quantize_rtn_int4(W, G, gi, sym=sym)
    q2, s2, z2 = int4.quantize_rtn_int4(W[:, perm], G, None, sym=sym)
    assert np.array_equal(q1[:, perm], q2) and np.array_equal(s1, s2)
    assert (z1 is None and z2 is None) if sym else np.array_equal(z1, z2)
