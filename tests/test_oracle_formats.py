"""Pins for the oracle's own number-format code (bf16 / fp16 decode and
round-to-nearest-even encode) against library conversions and the definition
of nearest-even rounding."""
import math

import numpy as np
import pytest
import torch

import oracle


def test_bf16_decode_all_patterns_match_torch():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.bf16_to_f64(bits)
    ref = torch.from_numpy(bits.view(np.int16)).view(torch.bfloat16).to(torch.float64).numpy()
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])
    # signed zeros decode with their sign
    assert math.copysign(1.0, ours[0x8000]) == -1.0


def test_fp16_decode_all_patterns_match_numpy():
    bits = np.arange(65536, dtype=np.uint32).astype(np.uint16)
    ours = oracle.f16_to_f64(bits)
    ref = bits.view(np.float16).astype(np.float64)
    nan = np.isnan(ref)
    assert np.array_equal(np.isnan(ours), nan)
    assert np.array_equal(ours[~nan], ref[~nan])


def _doubles(g, n):
    """Doubles across the fp16 / bf16 ranges, plus exact halfway cases."""
    mags = np.exp2(g.uniform(-30, 20, n))
    v = mags * np.where(g.random(n) < 0.5, -1.0, 1.0)
    return v


def test_fp16_encode_matches_numpy_nearest_even():
    g = np.random.default_rng(7)
    v = list(_doubles(g, 20000))
    # exact ties between fp16 neighbours: (2m+1) * 2^-11 near 1, subnormal ties,
    # the overflow threshold and its neighbours
    v += [1.0 + (2 * m + 1) * 2.0 ** -11 for m in range(64)]
    v += [(2 * m + 1) * 2.0 ** -25 for m in range(64)]
    v += [65504.0, 65519.99, 65520.0, 65536.0, 1e6, -65520.0, 0.0, -0.0, 2.0 ** -26]
    v = np.array(v)
    ours = oracle.f64_to_f16(v)
    ref = v.astype(np.float16).view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_matches_torch_on_float32_inputs():
    g = np.random.default_rng(8)
    v = _doubles(g, 20000).astype(np.float32)
    # exact ties: a float32 whose low 16 bits are 0x8000
    # (sign, exponent 2^-1..2^0, random 7-bit bf16 mantissa, then exactly half an ulp)
    m = g.integers(0, 128, 2000, dtype=np.uint32)
    sgn = g.integers(0, 2, 2000, dtype=np.uint32) << 31
    ex = (126 + g.integers(0, 2, 2000, dtype=np.uint32)) << 23
    tie = sgn | ex | (m << 16) | 0x8000
    v = np.concatenate([v, tie.astype(np.uint32).view(np.float32)])
    ours = oracle.f64_to_bf16(v.astype(np.float64))
    ref = torch.from_numpy(v).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(ours, ref)


def test_bf16_encode_is_nearest_even_on_doubles():
    """For doubles that are not float32 values, check the definition directly:
    the result is a nearest bf16 neighbour, and on an exact tie the even one."""
    g = np.random.default_rng(9)
    v = g.standard_normal(3000) * np.exp2(g.uniform(-20, 20, 3000))
    ours = oracle.f64_to_bf16(v)
    vals = oracle.bf16_to_f64(ours)
    for x, b, y in zip(v, ours, vals):
        up = oracle.bf16_to_f64(np.array([int(b) + 1], np.uint16))[0]
        dn = oracle.bf16_to_f64(np.array([int(b) - 1], np.uint16))[0]
        d = abs(x - y)
        assert d <= abs(x - up) and d <= abs(x - dn)
    # halfway between two bf16 values 1 + m/128 and 1 + (m+1)/128, exactly
    for m in range(20):
        x = 1.0 + (2 * m + 1) / 256.0
        y = oracle.bf16_to_f64(oracle.f64_to_bf16(np.array([x])))[0]
        lo, hi = 1.0 + m / 128.0, 1.0 + (m + 1) / 128.0
        assert y == (lo if m % 2 == 0 else hi)
