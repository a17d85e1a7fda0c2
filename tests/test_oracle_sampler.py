"""Pins for the oracle's keyed sampler.

* Gumbel-max is an exact draw: token frequencies match softmax(l/T) (chi-square
  on a 16-token vocabulary), and with top-k / top-p they match the renormalised
  truncated law, with exactly zero mass outside it.
* T -> 0: the noise is bounded, so a logit lead above (g_max - g_min) * T makes
  the argmax the sample for every seed; T == 0 is numpy's argmax.
* top-k / top-p selection equals brute-force enumeration on tiny vocabularies.
"""
import itertools
import math

import numpy as np
import pytest
from scipy import stats
from scipy.special import softmax

import oracle

CHI2_15_0001 = 37.697  # chi-square critical value, 15 dof, alpha = 0.001
G_WIDTH = 53 * math.log(2.0) + math.log(53 * math.log(2.0))  # g_max - g_min


def _chi2(counts, p):
    n = counts.sum()
    exp = n * p
    return float(((counts - exp) ** 2 / exp).sum())


@pytest.mark.parametrize("T", [0.5, 0.8, 1.0, 2.0])
def test_gumbel_max_frequencies_match_softmax_over_seeds_and_positions(T):
    g = np.random.default_rng(100 + int(T * 10))
    l = (g.standard_normal(16) * 1.5).astype(np.float32)
    p = softmax(l.astype(np.float64) / T)
    n = 200_000
    # over seeds at a fixed position
    tok = oracle.sample_many(l, np.full(n, 17, np.int64), np.arange(n, dtype=np.uint64),
                             T, 16, 1.0)
    assert _chi2(np.bincount(tok, minlength=16), p) < CHI2_15_0001
    # over positions at a fixed seed
    tok = oracle.sample_many(l, np.arange(n, dtype=np.int64), np.full(n, 42, np.uint64),
                             T, 16, 1.0)
    assert _chi2(np.bincount(tok, minlength=16), p) < CHI2_15_0001


def _truncated_law(l, T, k, top_p):
    order = sorted(range(len(l)), key=lambda i: (-float(l[i]), i))[:k]
    a = np.array([float(l[i]) for i in order]) / T
    e = np.exp(a - a[0])
    Z = e.sum()
    c = np.concatenate([[0.0], np.cumsum(e)])
    m = next(j for j in range(1, k + 1) if c[j] >= top_p * Z)
    keep = order[:m]
    pk = e[:m] / e[:m].sum()
    law = np.zeros(len(l))
    law[keep] = pk
    return law


@pytest.mark.parametrize("T,k,top_p", [(0.8, 8, 0.9), (1.0, 5, 0.95), (0.7, 16, 0.6)])
def test_truncated_frequencies_match_renormalised_law(T, k, top_p):
    g = np.random.default_rng(7 + k)
    l = (g.standard_normal(16) * 1.2).astype(np.float32)
    law = _truncated_law(l, T, k, top_p)
    n = 200_000
    tok = oracle.sample_many(l, np.full(n, 3, np.int64), np.arange(n, dtype=np.uint64),
                             T, k, top_p)
    cnt = np.bincount(tok, minlength=16)
    assert cnt[law == 0].sum() == 0
    sup = law > 0
    dof = int(sup.sum()) - 1
    if dof > 0:
        crit = stats.chi2.ppf(0.999, dof)
        assert _chi2(cnt[sup], law[sup]) < crit


def test_low_temperature_bound_makes_argmax_certain():
    g = np.random.default_rng(3)
    for trial in range(20):
        T = float(g.uniform(0.05, 2.0))
        l = (g.standard_normal(32) * 3).astype(np.float64)
        best = int(np.argmax(l))
        others = np.delete(l, best)
        l[best] = others.max() + (G_WIDTH + 0.01) * T
        l = l.astype(np.float32)
        assert (float(l[best]) - float(np.sort(l)[-2])) / T > G_WIDTH
        tok = oracle.sample_many(l, np.arange(500, dtype=np.int64),
                                 np.full(500, trial, np.uint64), T, 20, 1.0)
        assert np.all(tok == best)
    # just under the bound the argmax is not certain: some draws differ
    l = np.zeros(2, np.float32)
    l[0] = 2.0
    tok = oracle.sample_many(l, np.zeros(20000, np.int64), np.arange(20000, dtype=np.uint64),
                             1.0, 2, 1.0)
    assert 0 < (tok == 1).sum() < 20000


def test_greedy_is_numpy_argmax_lowest_index_on_ties():
    g = np.random.default_rng(11)
    for _ in range(50):
        V = int(g.integers(1, 300))
        l = g.integers(-5, 5, V).astype(np.float32)  # many ties
        o = oracle.sample_row(l, 0, 0.0, 20, 0.95, 1)
        assert o.token == int(np.argmax(l))
        if V > 1:
            s = np.sort(l)
            assert o.gap == float(s[-1]) - float(s[-2])
        else:
            assert math.isinf(o.gap)


def _brute_topk(l, k):
    """The k-subset whose every member ranks before every non-member under
    (logit desc, id asc)."""
    V = len(l)
    before = lambda a, b: l[a] > l[b] or (l[a] == l[b] and a < b)
    for sub in itertools.combinations(range(V), min(k, V)):
        rest = [i for i in range(V) if i not in sub]
        if all(before(a, b) for a in sub for b in rest):
            return set(sub)
    raise AssertionError


def _brute_nucleus(l, cand, T, top_p):
    """Smallest-cardinality subset of the candidates with mass >= top_p * Z; among
    equal sizes the one of largest mass (unique when logits are distinct)."""
    cand = list(cand)
    e = {i: math.exp((float(l[i]) - max(float(l[c]) for c in cand)) / T) for i in cand}
    Z = sum(e.values())
    for m in range(1, len(cand) + 1):
        best = None
        for sub in itertools.combinations(cand, m):
            mass = sum(e[i] for i in sub)
            if mass >= top_p * Z * (1 + 1e-12) and (best is None or mass > best[0]):
                best = (mass, set(sub))
        if best is not None:
            return best[1]
        # guard the rounding band: skip cases that sit on the boundary
        for sub in itertools.combinations(cand, m):
            if abs(sum(e[i] for i in sub) - top_p * Z) < 1e-9 * Z:
                return None
    return set(cand)


def test_topk_topp_selection_matches_brute_force():
    g = np.random.default_rng(5)
    checked = 0
    for trial in range(400):
        V = int(g.integers(2, 11))
        l = (g.standard_normal(V) * 2).astype(np.float32)
        if trial % 3 == 0:
            l[g.integers(0, V)] = l[0]  # a logit tie
        k = int(g.integers(1, V + 1))
        T = float(g.uniform(0.3, 2.0))
        top_p = float(g.uniform(0.2, 1.0))
        ids = oracle.topk(l, k)
        assert set(ids.tolist()) == _brute_topk(l, k)
        # the returned order is the total order itself
        assert all(l[a] > l[b] or (l[a] == l[b] and a < b) for a, b in zip(ids, ids[1:]))
        if len(set(l.tolist())) < V:
            continue
        nuc = _brute_nucleus(l, ids, T, top_p)
        if nuc is None:
            continue
        seed = int(g.integers(0, 1 << 62))
        pos = int(g.integers(0, 1000))
        o = oracle.sample_row(l, pos, T, k, top_p, seed)
        assert o.n_kept == len(nuc)
        z = {t: float(l[t]) / T + oracle.gumbel(oracle.noise_hash(seed, pos, t)) for t in nuc}
        assert o.token == max(sorted(nuc), key=lambda t: z[t])
        checked += 1
    assert checked > 150


def test_single_candidate_and_topk_one():
    l = np.array([0.1, 3.0, 3.0, -1.0], np.float32)
    o = oracle.sample_row(l, 0, 1.0, 1, 1.0, 9)
    assert o.token == 1 and math.isinf(o.gap) and o.n_kept == 1
    o = oracle.sample_row(l, 0, 1.0, 4, 1e-6, 9)  # tiny top_p keeps one
    assert o.token == 1 and o.n_kept == 1


# --- top-p over the whole vocabulary (top_k == 0) ---------------------------------

@pytest.mark.parametrize("T", [0.5, 1.0])
def test_no_topk_full_nucleus_frequencies_match_softmax(T):
    # top_k 0 and top_p 1: every token stays, the draw is softmax over all V
    g = np.random.default_rng(200 + int(T * 10))
    l = (g.standard_normal(16) * 1.5).astype(np.float32)
    p = softmax(l.astype(np.float64) / T)
    n = 100_000
    tok = oracle.sample_many(l, np.full(n, 5, np.int64), np.arange(n, dtype=np.uint64), T, 0, 1.0)
    assert _chi2(np.bincount(tok, minlength=16), p) < CHI2_15_0001


def _fixed_point_nucleus(l, T, top_p):
    """The nucleus by brute force over subsets: the smallest set of tokens
    whose fixed-point mass (nearest(exp((l - m) / T) * 2^40)) reaches the
    threshold trunc(top_p * Z), among equal sizes the heaviest (unique for
    distinct logits); None when a subset's mass sits within Z / 2^30 of it."""
    V = len(l)
    m = max(float(x) for x in l)
    e = [int(np.rint(math.exp((float(l[i]) - m) / T) * 2.0 ** 40)) for i in range(V)]
    Z = sum(e)
    thr = max(1, int(top_p * float(Z)))
    for size in range(1, V + 1):
        best = None
        for sub in itertools.combinations(range(V), size):
            mass = sum(e[i] for i in sub)
            if abs(mass - thr) < Z / 2 ** 30:
                return None
            if mass >= thr and (best is None or mass > best[0]):
                best = (mass, set(sub))
        if best is not None:
            return best[1]
    return set(range(V))


def test_no_topk_nucleus_matches_brute_force():
    g = np.random.default_rng(21)
    checked = 0
    for trial in range(300):
        V = int(g.integers(2, 10))
        l = (g.standard_normal(V) * 2).astype(np.float32)
        if len(set(l.tolist())) < V:
            continue
        T = float(g.uniform(0.3, 2.0))
        top_p = float(g.uniform(0.05, 1.0))
        nuc = _fixed_point_nucleus(l, T, top_p)
        if nuc is None:
            continue
        seed, pos = int(g.integers(0, 1 << 62)), int(g.integers(0, 1000))
        o = oracle.sample_row(l, pos, T, 0, top_p, seed)
        assert o.n_kept == len(nuc) and o.n_cand == V
        z = {t: float(l[t]) / T + oracle.gumbel(oracle.noise_hash(seed, pos, t)) for t in nuc}
        assert o.token == max(sorted(nuc), key=lambda t: z[t])
        checked += 1
    assert checked > 150


def test_no_topk_agrees_with_topk_of_the_whole_vocabulary_off_the_edge():
    # top_k = V keeps every token too; the two cuts read the masses in fp64 and
    # in fixed point, so they agree except at a cut within rounding of top_p Z
    g = np.random.default_rng(22)
    agree = 0
    for trial in range(200):
        V = int(g.integers(2, 65))
        l = (g.standard_normal(V) * 2).astype(np.float32)
        T, top_p = float(g.uniform(0.3, 2.0)), float(g.uniform(0.1, 1.0))
        seed, pos = int(g.integers(0, 1 << 62)), int(g.integers(0, 1000))
        a = oracle.sample_row(l, pos, T, 0, top_p, seed)
        b = oracle.sample_row(l, pos, T, V, top_p, seed)
        if a.topp_edge or b.topp_edge:
            continue
        assert (a.token, a.n_kept) == (b.token, b.n_kept)
        agree += 1
    assert agree > 180
