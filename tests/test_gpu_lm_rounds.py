"""The LM head + sampler workload end to end on the GPU: 64 hidden rows through
the W4 LM head (5120 -> 151936, G 64), then

* every (seed, position) pair of 1000 seeds x 64 positions sampled on the GPU
  (T 0.7, top-k 20, top-p 0.95) equals the oracle's draw from the same logits
  (the oracle's top-20 once per row, then its top-p and keyed argmax per
  pair), except where the oracle's decision sits in the last bits of fp64
  (top-two gap below 1e-12, or a top-p cut within 1e-9 Z), which are counted;
  greedy (T = 0) equals the oracle's argmax on every row;
* the logits match the oracle on sampled columns (per-row relative error);
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
from helpers import ROW_REL_TOL, dev, host, packed, row_rel_err

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


def _gpu_tokens(Ld, positions, seed, T_=T):
    return ev.keyed_sample(Ld, positions, T_, K_TOP, P_TOP, seed)


def test_logits_match_oracle_on_sampled_columns(lm):
    d, _, logits = lm
    q, s, b = d["w"]
    cols = np.unique(np.concatenate([np.arange(0, d["V"], 1499), [d["V"] - 1]]))
    ref = oracle.w4_linear(d["h"], q[cols], s[cols], b[cols], d["G"])
    err = row_rel_err(logits[:, cols], ref)
    assert np.all(err <= ROW_REL_TOL), err.max()


def test_thousand_seeds_by_sixty_four_positions(lm):
    _, _, logits = lm
    Ld = dev(logits)
    pos = torch.arange(N_POS, dtype=torch.int64, device="cuda")
    gpu = torch.empty((N_SEEDS, N_POS), dtype=torch.int32, device="cuda")
    for seed in range(N_SEEDS):
        for i in range(0, N_POS, 16):
            gpu[seed, i:i + 16] = _gpu_tokens(Ld[i:i + 16], pos[i:i + 16], seed)
    gpu = host(gpu)
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
