"""GPU parity of the NVFP4-style linear (verify_linear_nvfp4) against the
oracle: one-hot activations and small-integer activations with power-of-two
scales bit for bit; random cases (ragged shapes, both launch kinds) within the
2e-3 row tolerance; every row of an R-row call bit-identical to that row
alone; the packed layout against a numpy model of it."""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from helpers import ROW_REL_TOL, dev, host, row_rel_err

pytestmark = pytest.mark.gpu


def _packed(q, s, s_t):
    return ev.nvfp4_pack(dev(q), dev(s), s_t)


def _pack_codes(codes):
    codes = codes.astype(np.uint8)
    return (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)


def test_one_hot_reads_back_each_weight_bitwise():
    g = np.random.default_rng(1)
    N, K = 40, 256
    codes = g.integers(0, 16, (N, K))
    s = g.integers(0x08, 0x70, (N, K // 16)).astype(np.uint8)
    s_t = float(np.float32(0.37))
    w = _packed(_pack_codes(codes), s, s_t)
    ks = [0, 1, 3, 4, 15, 16, 17, 20, 31, 32, 127, 128, 200, 255]
    x = np.zeros((len(ks), K), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    xb = syn.bf16_bits(x)
    y = np.concatenate([host(ev.verify_linear_nvfp4(dev(xb[i:i + 16]), w)) for i in range(0, len(ks), 16)])
    ref = oracle.nvfp4_linear(xb, _pack_codes(codes), s, s_t)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


def test_exact_integer_case_bitwise():
    g = np.random.default_rng(2)
    R, N, K = 16, 300, 2048
    codes = g.integers(0, 16, (N, K))
    xi = g.integers(-3, 4, (R, K)).astype(np.float32)
    s = np.full((N, K // 16), 0x38, np.uint8)
    s[:, 1::2] = 0x40
    q = _pack_codes(codes)
    y = host(ev.verify_linear_nvfp4(dev(syn.bf16_bits(xi)), _packed(q, s, 1.0)))
    ref = oracle.nvfp4_linear(syn.bf16_bits(xi), q, s, 1.0)
    assert np.array_equal(y.view(np.uint32), ref.view(np.uint32))


@pytest.mark.parametrize("K,N", [(256, 512), (96, 33), (320, 40), (2048, 300), (5120, 1000), (4160, 17),
                                 (5120, 5000), (17408, 640)])
def test_random_parity_and_row_exactness(K, N):
    g = np.random.default_rng(K + N)
    q, s, s_t = syn.nvfp4_matrix(g, N, K)
    x = syn.activations(g, 16, K)
    w = _packed(q, s, s_t)
    y = host(ev.verify_linear_nvfp4(dev(x), w))
    ref = oracle.nvfp4_linear(x, q, s, s_t)
    err = row_rel_err(y, ref)
    assert np.all(err <= ROW_REL_TOL), err.max()
    for r in (0, 7, 15):
        y1 = host(ev.verify_linear_nvfp4(dev(x[r:r + 1]), w))
        assert np.array_equal(y1[0].view(np.uint32), y[r].view(np.uint32)), r
    for R in (2, 5):
        yR = host(ev.verify_linear_nvfp4(dev(x[:R]), w))
        assert np.array_equal(yR.view(np.uint32), y[:R].view(np.uint32))


def test_full_size_sampled_columns():
    g = np.random.default_rng(1010)
    for K, N in ((5120, 17408), (5120, 151936)):
        q, s, s_t = syn.nvfp4_matrix(g, N, K)
        x = syn.activations(g, 16, K)
        y = host(ev.verify_linear_nvfp4(dev(x), _packed(q, s, s_t)))
        cols = np.unique(np.concatenate([np.arange(0, N, 997), [N - 1]]))
        ref = oracle.nvfp4_linear(x, q[cols], s[cols], s_t)
        err = row_rel_err(y[:, cols], ref)
        assert np.all(err <= ROW_REL_TOL), (K, N, err.max())
        torch.cuda.empty_cache()


def test_packed_layout_model():
    g = np.random.default_rng(5)
    for N, K in ((32, 256), (17, 96), (40, 160)):
        codes = g.integers(0, 16, (N, K))
        s = g.integers(0, 256, (N, K // 16)).astype(np.uint8)
        blob = host(ev.nvfp4_pack(dev(_pack_codes(codes)), dev(s), 1.0).blob)
        T, C = -(-N // 16), -(-K // 128)
        assert blob.size == T * C * 1152
        for tile in range(T):
            for c in range(C):
                tc = blob[(c * T + tile) * 1152:(c * T + tile + 1) * 1152]
                for L in range(64):
                    ln, j = L % 16, L // 16
                    n = 16 * tile + ln
                    for t in range(4):
                        word = int.from_bytes(tc[16 * L + 4 * t:16 * L + 4 * t + 4].tobytes(), "little")
                        for e in range(8):
                            k = 128 * c + 32 * t + 4 * j + (e % 4) + 16 * (e // 4)
                            want = int(codes[n, k]) if n < N and k < K else 0
                            assert (word >> (4 * e)) & 15 == want, (N, K, tile, c, L, t, e)
                    if j == 0:
                        for b in range(8):
                            kb = 128 * c + 16 * b
                            want = int(s[n, kb // 16]) if n < N and kb < K else 0
                            assert tc[1024 + 8 * ln + b] == want
