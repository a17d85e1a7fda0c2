"""Pins for the accept rule (exhaustive enumeration against the rule stated as
"commit every sample up to and including the first one whose draft differs")
and for the MoE layer (routing against numpy / scipy, the layer against a
numpy reconstruction, and the single-dominant-expert reduction to one MLP)."""
import itertools

import numpy as np
import pytest
from scipy.special import softmax

import oracle
import synthetic as syn


def test_accept_exhaustive_small():
    for R in range(1, 5):
        for D in range(0, R + 1):
            for sampled in itertools.product(range(3), repeat=R):
                for draft in itertools.product(range(3), repeat=D):
                    a, n = oracle.accept(np.array(sampled), np.array(draft, dtype=np.int32))
                    mism = [i for i in range(D) if draft[i] != sampled[i]]
                    a_ref = mism[0] if mism else D
                    assert a == a_ref
                    # committed: samples 0..a (the first non-matching one included)
                    assert n == min(a_ref + 1, R)


def test_route_matches_numpy():
    g = np.random.default_rng(12)
    for trial in range(50):
        rho = g.standard_normal(128).astype(np.float32)
        if trial % 5 == 0:
            rho[10] = rho[20] = rho.max()  # tie at the top
        ids, w = oracle.moe_route(rho, 8)
        order = np.lexsort((np.arange(128), -rho.astype(np.float64)))[:8]
        assert np.array_equal(ids, order)
        p = softmax(rho.astype(np.float64))
        assert np.allclose(w, p[order] / p[order].sum(), rtol=1e-14)
        assert abs(w.sum() - 1.0) < 1e-14


def _small_moe(g, R=3, H=64, I=32, E=8, G=32):
    def stack(n, k):
        q = g.integers(0, 256, (E, n, k // 2), dtype=np.uint8)
        s = syn.fp16_bits(g.uniform(0.01, 0.05, (E, n, k // G)))
        b = syn.fp16_bits(g.normal(0, 0.1, (E, n, k // G)))
        return q, s, b
    return stack(I, H), stack(I, H), stack(H, I), syn.activations(g, R, H), \
        g.standard_normal((R, E)).astype(np.float32)


def _unpack(q):
    out = np.empty(q.shape[:-1] + (q.shape[-1] * 2,), np.int64)
    out[..., 0::2] = q & 15
    out[..., 1::2] = q >> 4
    return out


def _deq(q, s, b, G):
    sv = s.view(np.float16).astype(np.float64)
    bv = b.view(np.float16).astype(np.float64)
    return _unpack(q) * np.repeat(sv, G, axis=-1) + np.repeat(bv, G, axis=-1)


def test_moe_matches_numpy_reconstruction():
    g = np.random.default_rng(13)
    G, top = 32, 4
    gate, up, down, x, rho = _small_moe(g, G=G)
    y, ids, w = oracle.moe(x, rho, top, G, gate, up, down)
    xv = syn.bf16_values(x).astype(np.float64)
    for r in range(x.shape[0]):
        order = np.lexsort((np.arange(rho.shape[1]), -rho[r].astype(np.float64)))[:top]
        assert np.array_equal(ids[r], order)
        p = softmax(rho[r].astype(np.float64))[order]
        p /= p.sum()
        acc = np.zeros(x.shape[1])
        for j, e in enumerate(order):
            gg = (xv[r] @ _deq(*[a[e] for a in gate], G).T).astype(np.float32)
            uu = (xv[r] @ _deq(*[a[e] for a in up], G).T).astype(np.float32)
            hh = syn.bf16_values(oracle.silu_mul_bf16(gg, uu)).astype(np.float64)
            ye = (hh @ _deq(*[a[e] for a in down], G).T).astype(np.float32)
            acc += p[j] * ye
        assert np.max(np.abs(y[r] - acc)) <= 1e-6 * np.max(np.abs(acc))


def test_moe_with_one_dominant_expert_is_that_experts_mlp():
    g = np.random.default_rng(14)
    G = 32
    gate, up, down, x, rho = _small_moe(g, R=2, G=G)
    rho[:] = 0.0
    rho[0, 5] = 200.0
    rho[1, 2] = 200.0
    y, ids, w = oracle.moe(x, rho, 4, G, gate, up, down)
    for r, e in ((0, 5), (1, 2)):
        assert ids[r, 0] == e and w[r, 0] == 1.0
        ye, _, _, _ = oracle.mlp(x[r:r + 1], [a[e] for a in gate], [a[e] for a in up],
                                 [a[e] for a in down], G)
        assert np.array_equal(y[r], ye[0])
