"""Pins for the oracle's NVFP4-style linear (FP4 E2M1 elements, FP8 E4M3
block scales of 16, one fp32 tensor scale):

* E2M1 decode equals the OCP MX specification's FP4 table (tests/golden);
* E4M3 decode equals torch's float8_e4m3fn conversion for all 256 patterns;
* one-hot activations read back e2m1 * e4m3 * s_t exactly (nibble order and
  block index);
* small-integer activations with power-of-two scales: exact, bitwise against
  int64 arithmetic;
* random cases against numpy's float64 matmul on the dequantised matrix.
"""
import math
import os

import numpy as np
import torch

import oracle
import synthetic as syn

HERE = os.path.dirname(os.path.abspath(__file__))


def _e2m1_table():
    out = {}
    with open(os.path.join(HERE, "golden", "e2m1_values.txt")) as f:
        for line in f:
            if line.strip() and not line.startswith("#"):
                c, v = line.split()
                out[int(c)] = float(v)
    return out


def _e4m3(b):
    return torch.tensor(np.asarray(b, np.uint8)).view(torch.float8_e4m3fn).to(torch.float64).numpy()


def test_e2m1_matches_the_mx_table():
    t = _e2m1_table()
    assert len(t) == 16
    for c, v in t.items():
        got = oracle.e2m1_to_f64(c)
        assert got == v and math.copysign(1.0, got) == math.copysign(1.0, v), c


def test_e4m3_matches_torch_for_every_pattern():
    ref = _e4m3(np.arange(256))
    for b in range(256):
        got = oracle.e4m3_to_f64(b)
        if math.isnan(ref[b]):
            assert math.isnan(got), b
        else:
            assert got == ref[b] and math.copysign(1.0, got) == math.copysign(1.0, ref[b]), b


def _pack(codes):
    codes = codes.astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def _dequant(codes, sc, s_t):
    t = _e2m1_table()
    e = np.vectorize(lambda c: t[int(c)])(codes)
    return e * np.repeat(_e4m3(sc), 16, axis=1) * float(np.float32(s_t))


def test_one_hot_reads_back_one_weight():
    g = np.random.default_rng(1)
    N, K, s_t = 24, 128, np.float32(0.37)
    codes = g.integers(0, 16, (N, K))
    sc = g.integers(0, 0x7f, (N, K // 16)).astype(np.uint8)  # finite, positive
    ks = [0, 1, 2, 15, 16, 17, 31, 64, 126, 127]
    x = np.zeros((len(ks), K), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = oracle.nvfp4_linear(syn.bf16_bits(x), _pack(codes), sc, s_t)
    W = _dequant(codes, sc, s_t)
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], W[:, k].astype(np.float32))


def test_exact_integer_case_bitwise():
    g = np.random.default_rng(2)
    R, N, K = 3, 40, 256
    codes = g.integers(0, 16, (N, K))
    xi = g.integers(-3, 4, (R, K))
    sc = np.full((N, K // 16), 0x38, np.uint8)  # 1.0
    sc[:, 1::2] = 0x40                            # 2.0
    y = oracle.nvfp4_linear(syn.bf16_bits(xi.astype(np.float32)), _pack(codes), sc, 1.0)
    t = _e2m1_table()
    w2 = np.vectorize(lambda c: int(round(2 * t[int(c)])))(codes) * np.repeat(_e4m3(sc), 16, axis=1)
    ref = (xi.astype(np.int64) @ w2.T.astype(np.int64)).astype(np.float64) / 2.0
    assert np.array_equal(y, ref.astype(np.float32))


def test_random_matches_numpy_matmul():
    g = np.random.default_rng(3)
    for R, N, K in ((1, 7, 64), (4, 33, 512), (16, 40, 2048)):
        codes = g.integers(0, 16, (N, K))
        sc = g.integers(0x20, 0x50, (N, K // 16)).astype(np.uint8)
        s_t = np.float32(g.uniform(0.5, 2.0))
        x = syn.activations(g, R, K)
        y = oracle.nvfp4_linear(x, _pack(codes), sc, s_t)
        ref = syn.bf16_values(x).astype(np.float64) @ _dequant(codes, sc, s_t).T
        assert np.max(np.abs(y - ref)) <= 1e-6 * np.max(np.abs(ref))
