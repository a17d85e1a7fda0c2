"""The LM head + sampler workload end to end on the GPU: 64 hidden rows through
the W4 LM head (5120 -> 151936, G 64), then

* end to end: every (seed, position) pair of 1000 seeds x 64 positions drawn
  on the GPU from the GPU's logits (T 0.7, top-k 20, top-p 0.95) equals the
  oracle's draw from the oracle's own logits (its full LM head, every column),
  except where the oracle's two best perturbed scores differ by less than
  1e-4 (near ties) or its top-p cut lies within 1e-9 Z of a candidate's mass
  (top-p edges); both are counted and printed; greedy (T = 0) tokens equal
  the oracle's argmax except at logit gaps below 1e-4;
* the sampler alone: the same pairs drawn by the oracle from the GPU's logits
  agree except where the decision sits in the last bits of fp64 (gap below
  1e-12, or a top-p edge);
* the logits match the oracle's on every column (per-row relative error);
* the pages' sampling point (T 1, top-k 20, top-p 0.95, seeds 1234-1238)
  draws the oracle's token at all 64 positions;
* drafted rounds of R = 1, 2, 4, 8, 16 lanes slide over the 64 positions:
  lane r of a round at position p samples position p + r from hidden row
  p + r, the drafts for positions p .. p + R - 2 are the serial tokens with
  probability 0.7 (else a certainly wrong token), and accept_prefix commits
  min(accepted + 1, R) tokens.  The committed stream equals the serial one
  token for token for every R and seed, and the mean commit per round grows
  with R.
Seeded generators: synthetic.lm_head (1003) and synthetic.draft_coins.
"""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from helpers import NEAR_TIE, ROW_REL_TOL, dev, host, packed, row_rel_err

pytestmark = pytest.mark.gpu

T, K_TOP, P_TOP = 0.7, 20, 0.95
N_SEEDS, N_POS = 1000, 64


@pytest.fixture(scope="module")
def lm():
    d = syn.lm_head()
    wp = packed(d["w"], d["G"])
    H = d["h"]
    logits = np.concatenate([host(ev.verify_linear_w4(dev(H[i:i + 16]), wp)) for i in range(0, N_POS, 16)])
    yield d, wp, logits
    del wp
    torch.cuda.empty_cache()


@pytest.fixture(scope="module")
def oracle_logits(lm):
    d, _, _ = lm
    print("oracle LM head: 64 x 151936", flush=True)
    return oracle.w4_linear(d["h"], *d["w"], d["G"], out_f32=True)


def _gpu_tokens(Ld, positions, seed, T_=T):
    return ev.keyed_sample(Ld, positions, T_, K_TOP, P_TOP, seed)


def test_logits_match_oracle_on_every_column(lm, oracle_logits):
    _, _, logits = lm
    err = row_rel_err(logits, oracle_logits)
    print(f"LM head logits: max row error {err.max():.3e}")
    assert np.all(err <= ROW_REL_TOL), err.max()


def _gpu_grid(logits):
    Ld = dev(logits)
    pos = torch.arange(N_POS, dtype=torch.int64, device="cuda")
    gpu = torch.empty((N_SEEDS, N_POS), dtype=torch.int32, device="cuda")
    for seed in range(N_SEEDS):
        for i in range(0, N_POS, 16):
            gpu[seed, i:i + 16] = _gpu_tokens(Ld[i:i + 16], pos[i:i + 16], seed)
    return host(gpu)


def _cut_margins(row, cand, top_p):
    """How close the oracle's logits put a row's top-p cut and its top-k
    boundary to flipping: min over candidates j of |mass before j - top_p Z| / Z
    (fp64 masses e_j = exp((l_j - l_0) / T) in candidate order), and the
    logit gap between the k-th candidate and the best logit outside them."""
    l = row.astype(np.float64)
    lc = l[cand]
    e = np.exp((lc - lc[0]) / T)
    Z = e.sum()
    before = np.concatenate([[0.0], np.cumsum(e)[:-1]])
    topp = float(np.min(np.abs(before[1:] - top_p * Z)) / Z) if len(cand) > 1 else np.inf
    rest = np.delete(l, cand)
    topk = float(lc[-1] - rest.max()) if rest.size else np.inf
    return topp, topk


def test_thousand_seeds_by_sixty_four_positions_against_oracle_logits(lm, oracle_logits):
    """GPU tokens from GPU logits against oracle tokens from oracle logits.
    A difference is allowed only at an oracle decision within 1e-4 of
    flipping: the two best perturbed scores closer than 1e-4 (near tie), the
    top-p cut within 1e-4 Z of a candidate's mass (top-p edge), or the k-th
    and (k+1)-th logits closer than 1e-4 (top-k edge); each kind is counted."""
    _, _, logits = lm
    gpu = _gpu_grid(logits)
    near = edge_p = edge_k = 0
    for p in range(N_POS):
        cand = oracle.topk(oracle_logits[p], K_TOP)
        margins = None
        for seed in range(N_SEEDS):
            o = oracle.sample_from_candidates(oracle_logits[p], cand, p, T, P_TOP, seed)
            if o.token != gpu[seed, p]:
                if o.gap < NEAR_TIE:
                    near += 1
                    continue
                margins = margins or _cut_margins(oracle_logits[p], cand, P_TOP)
                if margins[0] < NEAR_TIE:
                    edge_p += 1
                elif margins[1] < NEAR_TIE:
                    edge_k += 1
                else:
                    raise AssertionError((seed, p, o.token, gpu[seed, p], o.gap, margins))
    print(f"{N_SEEDS} seeds x {N_POS} positions, tokens from the oracle's own logits: "
          f"{near} near-tie, {edge_p} top-p-edge, {edge_k} top-k-edge differences "
          f"of {N_SEEDS * N_POS} draws")
    # greedy: the GPU's argmax against the oracle's, lowest id on ties
    Ld = dev(logits)
    pos = torch.arange(N_POS, dtype=torch.int64, device="cuda")
    g = np.concatenate([host(_gpu_tokens(Ld[i:i + 16], pos[i:i + 16], 0, 0.0)) for i in range(0, N_POS, 16)])
    ref = np.argmax(oracle_logits, axis=1)
    top2 = np.sort(oracle_logits.astype(np.float64), axis=1)[:, -2:]
    gaps = top2[:, 1] - top2[:, 0]
    diff = g != ref
    assert np.all(gaps[diff] < NEAR_TIE), gaps[diff]
    print(f"greedy: {int(diff.sum())} of {N_POS} rows differ (all at logit gaps < 1e-4)")


def test_thousand_seeds_by_sixty_four_positions(lm):
    """The sampler alone: oracle draws from the GPU's own logits."""
    _, _, logits = lm
    gpu = _gpu_grid(logits)
    near = 0
    for p in range(N_POS):
        cand = oracle.topk(logits[p], K_TOP)
        for seed in range(N_SEEDS):
            o = oracle.sample_from_candidates(logits[p], cand, p, T, P_TOP, seed)
            if o.token != gpu[seed, p]:
                assert o.gap < 1e-12 or o.topp_edge, (seed, p, o.token, gpu[seed, p], o.gap)
                near += 1
    print(f"{N_SEEDS} seeds x {N_POS} positions: {near} decisions in the last bits of fp64")
    # greedy: the argmax of every row, lowest id on ties
    Ld = dev(logits)
    pos = torch.arange(N_POS, dtype=torch.int64, device="cuda")
    g = host(_gpu_tokens(Ld[:16], pos[:16], 0, 0.0))
    for i in range(16, N_POS, 16):
        g = np.concatenate([g, host(_gpu_tokens(Ld[i:i + 16], pos[i:i + 16], 0, 0.0))])
    assert np.array_equal(g, np.argmax(logits, axis=1).astype(np.int32))


def test_pages_sampling_point(lm):
    """The pages' own sampling setting (TensorFold README, the DGX Spark
    measurement after the CUDA engine paragraph: T 1, top-k 20, top-p 0.95,
    seeds 1234-1238, 64-token replies) on the same 64 hidden rows: every draw
    equals the oracle's, near-ties counted."""
    _, _, logits = lm
    Ld = dev(logits)
    pos = torch.arange(N_POS, dtype=torch.int64, device="cuda")
    near = 0
    for seed in range(1234, 1239):
        gpu = np.concatenate([host(_gpu_tokens(Ld[i:i + 16], pos[i:i + 16], seed, 1.0)) for i in range(0, N_POS, 16)])
        for p in range(N_POS):
            cand = oracle.topk(logits[p], K_TOP)
            o = oracle.sample_from_candidates(logits[p], cand, p, 1.0, P_TOP, seed)
            if o.token != gpu[p]:
                assert o.gap < 1e-12 or o.topp_edge, (seed, p, o.token, gpu[p], o.gap)
                near += 1
    print(f"seeds 1234-1238 x {N_POS} positions at T = 1: {near} decisions in the last bits of fp64")


@pytest.mark.parametrize("seed", [0, 17, 999])
def test_drafted_rounds_commit_the_serial_stream(lm, seed):
    d, wp, logits = lm
    V = d["V"]
    H = dev(d["h"])
    Ld = dev(logits)
    pos_all = torch.arange(N_POS, dtype=torch.int64, device="cuda")
    serial = np.concatenate([host(_gpu_tokens(Ld[i:i + 16], pos_all[i:i + 16], seed)) for i in range(0, N_POS, 16)])
    coins, offs = syn.draft_coins(seed, N_POS, 0.7)
    drafts = np.where(coins, serial, (serial + offs % (V - 1) + 1) % V).astype(np.int32)
    assert np.all((drafts == serial) == coins)
    mean_commit = {}
    for R in (1, 2, 4, 8, 16):
        p, rounds, committed = 0, 0, []
        while p < N_POS:
            Rr = min(R, N_POS - p)
            lg = ev.verify_linear_w4(H[p:p + Rr].contiguous(), wp)  # R-lane pass of the LM head
            s = ev.keyed_sample(lg, pos_all[p:p + Rr].contiguous(), T, K_TOP, P_TOP, seed)
            dr = dev(drafts[p:p + Rr - 1]) if Rr > 1 else None
            a, n = ev.accept_prefix(s, dr)
            n = int(host(n)[0])
            sh = host(s)
            ra, rn = oracle.accept(sh, drafts[p:p + Rr - 1])
            assert (int(host(a)[0]), n) == (ra, rn)
            committed.extend(sh[:n].tolist())
            p += n
            rounds += 1
        assert committed == serial.tolist(), R
        mean_commit[R] = N_POS / rounds
    print(f"seed {seed}: mean commit per round", {r: round(v, 2) for r, v in mean_commit.items()})
    assert mean_commit[1] == 1.0
    assert mean_commit[16] > mean_commit[2] > 1.0
