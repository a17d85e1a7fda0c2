"""Pins for the oracle's W4 linear and MLP glue.

* exact-integer case: every product and partial sum is an exact binary
  fraction, so the result must equal numpy int64 arithmetic bit for bit;
* one-hot activations read back a single dequantised weight, pinning nibble
  order and group indexing against a packing done here;
* random cases against numpy's float64 matmul on the dequantised matrix;
* SiLU against scipy's logistic function, the MLP against numpy end to end.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import synthetic as syn


def _pack(qv):
    """Pack codes [N][K] (0..15) two per byte, even k in the low nibble."""
    qv = qv.astype(np.uint8)
    return (qv[:, 0::2] | (qv[:, 1::2] << 4)).astype(np.uint8)


def _dequant(qv, s_bits, b_bits, G):
    s = s_bits.view(np.float16).astype(np.float64)
    b = b_bits.view(np.float16).astype(np.float64)
    return qv * np.repeat(s, G, axis=1) + np.repeat(b, G, axis=1)


@pytest.mark.parametrize("G", [32, 64])
def test_exact_integer_case_bitwise(G):
    g = np.random.default_rng(1)
    R, K, N = 3, 256, 40
    qv = g.integers(0, 16, (N, K))
    xi = g.integers(-3, 4, (R, K))
    bi = g.integers(-8, 9, (N, K // G))
    x = syn.bf16_bits(xi.astype(np.float32))
    s = syn.fp16_bits(np.full((N, K // G), 2.0 ** -5))
    b = syn.fp16_bits(bi * 2.0 ** -10)
    y = oracle.w4_linear(x, _pack(qv), s, b, G)
    # 1024 * y = sum_k x * (32 q + b_int), all in int64
    w_int = 32 * qv + np.repeat(bi, G, axis=1)
    ref = (xi.astype(np.int64) @ w_int.T.astype(np.int64)).astype(np.float64) / 1024.0
    assert np.array_equal(y, ref)
    y32 = oracle.w4_linear(x, _pack(qv), s, b, G, out_f32=True)
    assert np.array_equal(y32, ref.astype(np.float32))


@pytest.mark.parametrize("G", [32, 64])
def test_one_hot_reads_back_one_weight(G):
    g = np.random.default_rng(2)
    K, N = 128, 24
    qv = g.integers(0, 16, (N, K))
    s = syn.fp16_bits(g.uniform(0.01, 0.05, (N, K // G)))
    b = syn.fp16_bits(g.normal(0, 0.1, (N, K // G)))
    ks = [0, 1, 2, 31, 32, 33, G - 1, G, K - 2, K - 1]
    x = np.zeros((len(ks), K), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = oracle.w4_linear(syn.bf16_bits(x), _pack(qv), s, b, G)
    W = _dequant(qv, s, b, G)
    for r, k in enumerate(ks):
        assert np.array_equal(y[r], W[:, k])


@pytest.mark.parametrize("R,K,N,G", [(1, 64, 7, 64), (4, 256, 512, 64), (5, 96, 33, 32),
                                     (16, 320, 40, 32)])
def test_random_matches_numpy_matmul(R, K, N, G):
    g = np.random.default_rng(R * 1000 + K)
    qv = g.integers(0, 16, (N, K))
    s = syn.fp16_bits(g.uniform(0.01, 0.05, (N, K // G)))
    b = syn.fp16_bits(g.normal(0, 0.1, (N, K // G)))
    x = syn.activations(g, R, K)
    y = oracle.w4_linear(x, _pack(qv), s, b, G)
    ref = syn.bf16_values(x).astype(np.float64) @ _dequant(qv, s, b, G).T
    assert np.max(np.abs(y - ref)) <= 1e-12 * np.max(np.abs(ref))


def test_silu_matches_scipy_logistic():
    v = np.concatenate([np.linspace(-40, 40, 2001), [0.0, 1e-30, -1e-30, 700.0, -700.0]])
    ours = np.array([oracle.silu(float(t)) for t in v])
    ref = v * expit(v)
    assert np.allclose(ours, ref, rtol=1e-14, atol=1e-300)
    assert oracle.silu(0.0) == 0.0


def test_silu_mul_rounds_to_nearest_bf16():
    g = np.random.default_rng(4)
    a = (g.standard_normal(5000) * 3).astype(np.float32)
    c = (g.standard_normal(5000) * 3).astype(np.float32)
    h = oracle.silu_mul_bf16(a, c)
    exact = a.astype(np.float64) * expit(a.astype(np.float64)) * c.astype(np.float64)
    hv = syn.bf16_values(h).astype(np.float64)
    # nearest bf16: within half a bf16 ulp (2^-8 relative) of the exact product
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(exact), 1e-38))) - 7)
    assert np.all(np.abs(hv - exact) <= 0.5 * ulp * (1 + 1e-9))


def test_mlp_matches_numpy():
    g = np.random.default_rng(6)
    R, H, I, G = 3, 128, 192, 64
    mats = []
    for n, k in ((I, H), (I, H), (H, I)):
        qv = g.integers(0, 16, (n, k))
        mats.append((qv, syn.fp16_bits(g.uniform(0.01, 0.05, (n, k // G))),
                     syn.fp16_bits(g.normal(0, 0.1, (n, k // G)))))
    x = syn.activations(g, R, H)
    packed = [(_pack(q), s, b) for q, s, b in mats]
    y, gg, uu, h = oracle.mlp(x, packed[0], packed[1], packed[2], G)
    xv = syn.bf16_values(x).astype(np.float64)
    Wg, Wu, Wd = (_dequant(q, s, b, G) for q, s, b in mats)
    g_ref = (xv @ Wg.T).astype(np.float32)
    u_ref = (xv @ Wu.T).astype(np.float32)
    assert np.max(np.abs(gg - g_ref)) <= 1e-6 * np.max(np.abs(g_ref))
    assert np.max(np.abs(uu - u_ref)) <= 1e-6 * np.max(np.abs(u_ref))
    hv = syn.bf16_values(h).astype(np.float64)
    h_exact = g_ref * expit(g_ref.astype(np.float64)) * u_ref
    assert np.max(np.abs(hv - h_exact)) <= 2.0 ** -8 * np.max(np.abs(h_exact))
    y_ref = hv @ Wd.T
    assert np.max(np.abs(y - y_ref)) <= 1e-6 * np.max(np.abs(y_ref))


# --- the fp32 two-level evaluation (oracle.w4_linear_fp32) ---------------------

@pytest.mark.parametrize("G", [32, 64])
def test_fp32_mode_exact_integer_case_bitwise(G):
    # every fp32 product, dequantised weight and partial sum is exact here
    g = np.random.default_rng(11)
    R, K, N = 4, 256, 33
    qv = g.integers(0, 16, (N, K))
    xi = g.integers(-3, 4, (R, K))
    bi = g.integers(-8, 9, (N, K // G))
    x = syn.bf16_bits(xi.astype(np.float32))
    s = syn.fp16_bits(np.full((N, K // G), 2.0 ** -5))
    b = syn.fp16_bits(bi * 2.0 ** -10)
    y = oracle.w4_linear_fp32(x, _pack(qv), s, b, G)
    w_int = 32 * qv + np.repeat(bi, G, axis=1)
    ref = (xi.astype(np.int64) @ w_int.T.astype(np.int64)).astype(np.float64) / 1024.0
    assert np.array_equal(y, ref.astype(np.float32))


@pytest.mark.parametrize("G", [32, 64])
def test_fp32_mode_one_hot_reads_back_fp32_dequant(G):
    # y = fl32(fl32(s * q) + b): one product and one sum in binary32
    g = np.random.default_rng(12)
    K, N = 128, 24
    qv = g.integers(0, 16, (N, K))
    s = syn.fp16_bits(g.uniform(0.01, 0.05, (N, K // G)))
    b = syn.fp16_bits(g.normal(0, 0.1, (N, K // G)))
    ks = [0, 1, 31, 32, G - 1, G, K - 1]
    x = np.zeros((len(ks), K), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    y = oracle.w4_linear_fp32(syn.bf16_bits(x), _pack(qv), s, b, G)
    sv = s.view(np.float16).astype(np.float32)
    bv = b.view(np.float16).astype(np.float32)
    for r, k in enumerate(ks):
        w = (sv[:, k // G] * qv[:, k].astype(np.float32)).astype(np.float32) + bv[:, k // G]
        assert np.array_equal(y[r], w.astype(np.float32))


@pytest.mark.parametrize("R,K,N,G", [(2, 256, 64, 64), (3, 5120, 40, 64), (2, 2048, 32, 32)])
def test_fp32_mode_within_its_rounding_bound_of_fp64(R, K, N, G):
    # Every fp32 step rounds once (relative 2^-24): the dequantised weight
    # twice, each product once, a group's recursive sum at most G - 1 times and
    # the sum over groups K/G - 1 times, so |y32 - y| <= (G + K/G + 2) 2^-24
    # sum_k |w x| to first order (the factor 1.01 covers the higher orders).
    g = np.random.default_rng(K + N)
    qv = g.integers(0, 16, (N, K))
    s = syn.fp16_bits(g.uniform(0.01, 0.05, (N, K // G)))
    b = syn.fp16_bits(g.normal(0, 0.1, (N, K // G)))
    x = syn.activations(g, R, K)
    y32 = oracle.w4_linear_fp32(x, _pack(qv), s, b, G).astype(np.float64)
    y64 = oracle.w4_linear(x, _pack(qv), s, b, G)
    absum = np.abs(syn.bf16_values(x).astype(np.float64)) @ np.abs(_dequant(qv, s, b, G)).T
    bound = 1.01 * (G + K // G + 2) * 2.0 ** -24 * absum
    assert np.all(np.abs(y32 - y64) <= bound)
    # and far inside the 2e-3 row tolerance the GPU is held to
    rel = np.max(np.abs(y32 - y64), axis=1) / np.max(np.abs(y64), axis=1)
    assert np.all(rel < 1e-4)
