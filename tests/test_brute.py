"""The brute force's own bit decoding against numpy's converters (every 16-bit
pattern, and a sweep of fp32 patterns including the special classes)."""

import math

import numpy as np

import brute


def _same(a: float, b: float) -> bool:
    return (math.isnan(a) and math.isnan(b)) or (a == b and math.copysign(1, a) == math.copysign(1, b))


def test_decode_bits_f16_all_patterns():
    ref = np.arange(1 << 16, dtype=np.uint32).astype(np.uint16).view(np.float16).astype(np.float64)
    assert all(_same(brute.decode_bits(b, "f16"), float(ref[b])) for b in range(1 << 16))


def test_decode_bits_bf16_all_patterns():
    ref = (np.arange(1 << 16, dtype=np.uint32) << 16).view(np.float32).astype(np.float64)
    assert all(_same(brute.decode_bits(b, "bf16"), float(ref[b])) for b in range(1 << 16))


def test_decode_bits_f32_sweep():
    rng = np.random.Generator(np.random.PCG64(7))
    pats = np.concatenate([rng.integers(0, 1 << 32, 20000, dtype=np.uint64).astype(np.uint32),
                           np.array([0, 1, 0x007FFFFF, 0x00800000, 0x7F7FFFFF, 0x7F800000, 0x7FC00000,
                                     0x80000000, 0x80000001, 0xFF800000, 0xFFFFFFFF], np.uint32)])
    ref = pats.view(np.float32).astype(np.float64)
    assert all(_same(brute.decode_bits(int(b), "f32"), float(r)) for b, r in zip(pats, ref))
