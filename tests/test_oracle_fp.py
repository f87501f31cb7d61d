"""Pins for oracle/fp.py against independent library rounding routines."""

import struct

import numpy as np
import torch

from oracle import fp


def _torch_bf16_bits(a32):
    t = torch.from_numpy(np.ascontiguousarray(a32, dtype=np.float32)).to(torch.bfloat16)
    return t.view(torch.int16).numpy().view(np.uint16)


def test_bf16_rounding_matches_torch_random():
    r = np.random.default_rng(1)
    bits = r.integers(0, 2**32, size=200_000, dtype=np.uint64).astype(np.uint32)
    a = bits.view(np.float32)
    a = a[np.isfinite(a)]
    assert np.array_equal(fp.f32_to_bf16_bits(a), _torch_bf16_bits(a))


def test_bf16_rounding_ties_and_specials():
    # low half exactly 0x8000 is a tie: rounds to the even kept pattern
    hi = np.arange(0, 0x7F80, 37, dtype=np.uint32)
    ties = ((hi << 16) | 0x8000).view(np.float32)
    got = fp.f32_to_bf16_bits(ties)
    want = np.where(hi % 2 == 0, hi, hi + 1).astype(np.uint16)
    assert np.array_equal(got, want)
    specials = np.array([0.0, -0.0, np.inf, -np.inf, 3.4028235e38, 1e-45, -1e-45,
                         1.1754942e-38], dtype=np.float32)
    assert np.array_equal(fp.f32_to_bf16_bits(specials), _torch_bf16_bits(specials))
    nan = fp.f32_to_bf16_bits(np.array([np.nan], dtype=np.float32))
    assert (nan[0] & 0x7F80) == 0x7F80 and (nan[0] & 0x7F) != 0


def test_bf16_widen_is_exact():
    b = np.arange(0, 2**16, dtype=np.uint32).astype(np.uint16)
    w = fp.bf16_bits_to_f32(b)
    finite = np.isfinite(w)
    assert np.array_equal(fp.f32_to_bf16_bits(w[finite]), b[finite])


def test_f16_rounding_matches_struct_pack():
    # Python's struct 'e' packing rounds to nearest, ties to even
    r = np.random.default_rng(2)
    a = (r.standard_normal(20_000) * np.exp(r.uniform(-20, 10, 20_000))).astype(np.float32)
    a = a[np.abs(a) < 65504]
    got = fp.round_to(a, "f16")
    want = np.array([struct.unpack("<H", struct.pack("<e", float(v)))[0] for v in a],
                    dtype=np.uint16)
    assert np.array_equal(got, want)
