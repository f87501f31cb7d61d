"""Pins for oracle/intb.py (3-, 4- and 8-bit codes) and the b-bit repack layouts:
exhaustive bit positions, agreement with the separately written 4-bit oracle,
exact grid recovery, brute-force nearest levels, exact dequant, bijection and
addressing of the tiles."""

import struct
from fractions import Fraction

import numpy as np
import pytest
import torch

from oracle import intb, int4, repack, gemm, fp
from bit_weight_only_gemm_amd import synth


def _stream(words):
    """The little-endian integer of a run of words (one column)."""
    return sum(int(w) << (32 * i) for i, w in enumerate(np.asarray(words).view(np.uint32)))


# ---------------------------------------------------------------- packing

def test_pack3_every_position_and_value():
    # a single code v at position e of a 32-code run is the stream v << 3e,
    # including the codes that straddle words (e = 10: bits 30..32, e = 21:
    # bits 63..65)
    for e in range(32):
        for v in range(8):
            q = np.zeros((1, 32), dtype=np.uint8)
            q[0, e] = v
            w = intb.pack_qweight(q, 3)
            assert w.shape == (3, 1)
            assert _stream(w[:, 0]) == v << (3 * e), (e, v)
            assert np.array_equal(intb.unpack_qweight(w, 3), q)


def test_pack8_bytes_little_endian():
    q = np.arange(8, dtype=np.uint8).reshape(1, 8) * 31
    w = intb.pack_qweight(q, 8).view(np.uint32)
    assert w.shape == (2, 1)
    assert int(w[0, 0]) == int.from_bytes(bytes(q[0, :4]), "little")
    assert int(w[1, 0]) == int.from_bytes(bytes(q[0, 4:]), "little")


def test_pack4_equals_int4_oracle():
    r = np.random.default_rng(50)
    q = r.integers(0, 16, size=(24, 256)).astype(np.uint8)
    z = r.integers(0, 16, size=(2, 24)).astype(np.uint8)
    assert np.array_equal(intb.pack_qweight(q, 4), int4.pack_qweight(q))
    assert np.array_equal(intb.pack_qzeros(z, 4), int4.pack_qzeros(z))


@pytest.mark.parametrize("bits", [3, 8])
def test_pack_roundtrip_random(bits):
    r = np.random.default_rng(51 + bits)
    q = r.integers(0, 1 << bits, size=(64, 512)).astype(np.uint8)
    z = r.integers(0, 1 << bits, size=(4, 64)).astype(np.uint8)
    w = intb.pack_qweight(q, bits)
    assert w.dtype == np.int32 and w.shape == (512 * bits // 32, 64)
    assert np.array_equal(intb.unpack_qweight(w, bits), q)
    wz = intb.pack_qzeros(z, bits)
    assert wz.shape == (4, 64 * bits // 32)
    assert np.array_equal(intb.unpack_qzeros(wz, bits), z)


def test_pack3_zeros_run_along_n():
    z = np.zeros((1, 32), dtype=np.uint8)
    z[0, 21] = 5                      # bits 63..65: straddles words 1 and 2
    w = intb.pack_qzeros(z, 3)
    assert _stream(w[0]) == 5 << 63


# --------------------------------------------------------------- quantizer

@pytest.mark.parametrize("bits", [3, 8])
@pytest.mark.parametrize("G", [32, 128])
def test_rtn_recovers_exact_grid(bits, G):
    # w = (q - z) s with codes 0 and 2^b - 1 in every (row, group): the
    # quantizer returns q, s, z exactly (a wrong level count or group shows)
    N, K = 6, 512
    qmax = (1 << bits) - 1
    r = np.random.default_rng(60 + bits + G)
    ng = K // G
    s = r.uniform(0.001, 0.02, size=(ng, N)).astype(np.float16).astype(np.float32)
    z = r.integers(0, qmax + 1, size=(ng, N))
    q = r.integers(0, qmax + 1, size=(N, K))
    for g in range(ng):
        q[:, g * G] = 0
        q[:, g * G + 1] = qmax
    gk = np.arange(K) // G
    W = ((q - z[gk].T) * s[gk].T).astype(np.float32)
    q2, s2, z2 = intb.quantize_rtn(W, bits, G)
    assert np.array_equal(q2, q) and np.array_equal(z2, z)
    assert np.array_equal(s2.astype(np.float32), s)


@pytest.mark.parametrize("bits", [3, 8])
def test_symmetric_rtn_recovers_exact_grid(bits):
    N, K, G = 5, 256, 64
    h = intb.sym_zero(bits)
    r = np.random.default_rng(70 + bits)
    s = r.uniform(0.001, 0.02, size=(K // G, N)).astype(np.float16).astype(np.float32)
    c = r.integers(-(h - 1), h, size=(N, K))
    c[:, ::G] = h - 1                  # max |w| = (2^(b-1) - 1) s in every group
    gk = np.arange(K) // G
    W = (c * s[gk].T).astype(np.float32)
    q, s2, z = intb.quantize_rtn(W, bits, G, sym=True)
    assert z is None
    assert np.array_equal(q.astype(np.int64), c + h)
    assert np.array_equal(s2.astype(np.float32), s)


@pytest.mark.parametrize("bits", [3, 8])
@pytest.mark.parametrize("sym", [False, True])
def test_rtn_nearest_level_brute_force(bits, sym):
    G = 64
    W = synth.weights("test/intb/brute/%d/%d" % (bits, sym), 4, 256)
    q, s, z = intb.quantize_rtn(W, bits, G, sym=sym)
    for n in range(4):
        for k in range(0, 256, 3):
            g = k // G
            sf = np.float64(s[g, n])
            zz = intb.sym_zero(bits) if sym else int(z[g, n])
            levels = (np.arange(1 << bits) - zz) * sf
            d = np.abs(levels - np.float64(W[n, k]))
            assert d[q[n, k]] <= d.min() + 1e-6 * sf


@pytest.mark.parametrize("sym", [False, True])
def test_rtn4_equals_int4_oracle(sym):
    W = synth.weights("test/intb/eq4/%d" % sym, 16, 512)
    gi = synth.act_order_gidx("test/intb/eq4/g", 512, 64)
    a = intb.quantize_rtn(W, 4, 64, gi, sym=sym)
    b = int4.quantize_rtn_int4(W, 64, gi, sym=sym)
    for u, v in zip(a, b):
        assert (u is None and v is None) or np.array_equal(u, v)


@pytest.mark.parametrize("bits", [3, 8])
def test_symmetric_rtn_is_odd(bits):
    W = synth.weights("test/intb/odd/%d" % bits, 8, 256)
    h = intb.sym_zero(bits)
    q1, s1, _ = intb.quantize_rtn(W, bits, 32, sym=True)
    q2, s2, _ = intb.quantize_rtn(-W, bits, 32, sym=True)
    assert q1.min() >= 1
    assert np.array_equal(q2.astype(np.int64), 2 * h - q1.astype(np.int64))
    assert np.array_equal(s1, s2)


# ----------------------------------------------------------------- dequant

def _f16_of_exact(v):
    if abs(v) >= 65520.0:
        return int(np.float16(np.inf if v > 0 else -np.inf).view(np.uint16))
    return struct.unpack("<H", struct.pack("<e", v))[0]


@pytest.mark.parametrize("dtype", ["f16", "bf16"])
def test_dequant8_exhaustive_differences_vs_exact(dtype):
    # every q - z in [-255, 255] against a spread of scales
    scales = np.array([2.0**-24, 2.0**-14, 0.001, 0.0173, 0.5, 1.0, 3.0, 255.0, 60000.0],
                      dtype=np.float16)
    q = np.tile(np.arange(256, dtype=np.uint8), (len(scales), 2))[:, :512]
    N, K = len(scales), 512
    zeros = np.array([[0] * N, [255] * N], dtype=np.uint8)            # groups of 256
    s = np.tile(scales[None, :], (2, 1))
    got = intb.dequant_codes(q, s, zeros, 8, None, 256, dtype)
    for n in range(N):
        for k in range(0, K, 5):
            g = k // 256
            exact = Fraction(int(q[n, k]) - int(zeros[g, n])) * Fraction(float(scales[n]))
            if dtype == "f16":
                want = _f16_of_exact(float(exact))
            else:
                t = torch.tensor([float(exact)], dtype=torch.float64).to(torch.bfloat16)
                want = int(t.view(torch.int16).numpy().view(np.uint16)[0])
            if exact == 0:
                want = 0
            assert int(got[n, k]) == want, (n, k, dtype)


@pytest.mark.parametrize("bits", [3, 8])
def test_symmetric_dequant_zero_and_mirror(bits):
    h = intb.sym_zero(bits)
    q = np.arange(1 << bits, dtype=np.uint8)[None, :].repeat(2, 0)
    K = q.shape[1]
    K32 = max(K, 32)
    q = np.pad(q, ((0, 0), (0, K32 - K)), constant_values=h)
    s = np.array([[0.37, 0.0125]], dtype=np.float16)
    w = intb.dequant_codes(q, s, None, bits, None, K32, "f16")
    assert np.all(w[:, h] == 0)
    for d in range(1, h):
        assert np.all(w[:, h + d] ^ w[:, h - d] == 0x8000)


@pytest.mark.parametrize("bits", [3, 8])
def test_quantized_product_within_closed_form_bound(bits):
    M, N, K, G = 3, 16, 512, 64
    W = synth.weights("test/intb/bound/%d" % bits, N, K)
    x = synth.to_f16_bits(synth.activations("test/intb/bound/x/%d" % bits, M, K))
    q, s, z = intb.quantize_rtn(W, bits, G)
    wd = intb.dequant_codes(q, s, z, bits, None, G, "f16")
    xf = fp.bits_to_f64(x, "f16")
    y_ref = gemm.gemm_ref_bits(x, wd, "f16")
    y_flt = gemm.gemm_ref_fp64(xf, W.astype(np.float64))
    sk = s.astype(np.float64)[np.arange(K) // G].T
    qmax = (1 << bits) - 1
    per_w = sk * (0.5 + qmax * 2.0**-11) + 2.0**-11 * np.abs(fp.bits_to_f64(wd, "f16")) + 1e-12
    assert np.all(np.abs(y_ref - y_flt) <= np.abs(xf) @ per_w.T)


# ------------------------------------------------------------ repack layouts

@pytest.mark.parametrize("bits", [3, 8])
@pytest.mark.parametrize("G,sym,act", [(128, False, False), (32, True, True), (64, False, True),
                                       (256, True, False), (1280, False, False)])
def test_repack_bits_bijection(bits, G, sym, act):
    K, N = 1280, 224
    W = synth.weights("test/intb/rp/%d/%d" % (bits, G), N, K)
    gi = synth.act_order_gidx("test/intb/rp/g/%d" % G, K, G) if act else None
    q, s, z = intb.quantize_rtn(W, bits, G, gi, sym)
    cr, sr, zr, perm = repack.repack_ref_bits(intb.pack_qweight(q, bits), s,
                                              None if sym else intb.pack_qzeros(z, bits), bits,
                                              gi, G)
    U = repack.units_per_tile(G)
    NP, KT = (N + 63) // 64, K // 128
    KT8 = (KT + 7) // 8
    assert cr.size == NP * KT * 4 * 256 * bits
    assert sr.size == NP * KT8 * 512 * U
    if not sym:
        assert zr.size == NP * KT8 * 64 * U * (2 if bits == 8 else 1)
    q2, s2, z2 = repack.unrepack_ref_bits(cr, sr, zr, K, N, bits, G)
    qp = q if perm is None else q[:, perm]
    assert np.array_equal(q2, qp) and np.array_equal(s2, s)
    assert (z2 is None) if sym else np.array_equal(z2, z)


def test_repack4_bits_equals_repack_ref():
    K, N, G = 1024, 200, 64
    W = synth.weights("test/intb/rp4", N, K)
    q, s, z = int4.quantize_rtn_int4(W, G)
    a = repack.repack_ref(int4.pack_qweight(q), s, int4.pack_qzeros(z), None, G)
    b = repack.repack_ref_bits(intb.pack_qweight(q, 4), s, intb.pack_qzeros(z, 4), 4, None, G)
    for u, v in zip(a[:3], b[:3]):
        assert np.array_equal(u, v)


@pytest.mark.parametrize("bits", [3, 8])
def test_repack_bits_single_code_addressing(bits):
    # one code lands at the documented dword and bit(s) of the documented lane
    K, N, G = 256, 128, 128
    rr = np.random.default_rng(80 + bits)
    top = (1 << bits) - 1
    tile = 256 * bits                                  # bytes per (column tile, K tile)
    for _ in range(40):
        n, k = int(rr.integers(N)), int(rr.integers(K))
        v = int(rr.integers(1, top + 1))
        q = np.zeros((N, K), dtype=np.uint8)
        q[n, k] = v
        cr, _, _, _ = repack.repack_ref_bits(intb.pack_qweight(q, bits),
                                             np.zeros((K // G, N), np.float16), None, bits)
        p, c, i = n // 64, (n % 64) // 16, n % 16
        t, j, b, e = k // 128, (k % 128) // 32, (k % 32) // 8, k % 8
        lane = i + 16 * b
        base = ((p * (K // 128) + t) * 4 + c) * tile
        words = cr.view(np.uint32)
        if bits == 8:
            h = j >> 1
            d = 2 * (j & 1) + (e >> 2)
            off = base + h * 1024 + lane * 16 + 4 * d
            slot = ((e & 3) >> 1) + 2 * (e & 1)
            assert int(words[off // 4]) == v << (8 * slot)
            assert np.count_nonzero(words) == 1
        else:
            off = base + lane * 12
            lo = v & 3
            hi = v >> 2
            want = {}
            if lo:
                want[off // 4 + (j >> 1)] = lo << (16 * (e & 1) + 2 * (4 * (j & 1) + (e >> 1)))
            if hi:
                want[off // 4 + 2] = 1 << (16 * (e & 1) + 4 * j + (e >> 1))
            nz = {int(ix): int(words[ix]) for ix in np.nonzero(words)[0]}
            assert nz == want, (n, k, v)


def test_repack8_zero_addressing():
    K, N, G = 2048, 128, 64
    KT, U = K // 128, repack.units_per_tile(G)
    KT8 = (KT + 7) // 8
    rr = np.random.default_rng(90)
    for _ in range(12):
        n, g = int(rr.integers(N)), int(rr.integers(K // G))
        z = np.zeros((K // G, N), np.uint8)
        z[g, n] = 0xA7
        _, _, zr, _ = repack.repack_ref_bits(intb.pack_qweight(np.zeros((N, K), np.uint8), 8),
                                             np.zeros((K // G, N), np.float16),
                                             intb.pack_qzeros(z, 8), 8, None, G)
        p, c, i = n // 64, (n % 64) // 16, n % 16
        run, r = g // (8 * U), g % (8 * U)
        base = ((p * KT8 + run) * 4 + c) * 16 + i
        assert zr[base * 2 * U + r // 4] == 0xA7 << (8 * (r % 4))
        assert np.count_nonzero(zr) == 1
