"""Host round loop (no GPU): the commit rule and next position on a scripted
verify pass, the fallback to one row a round when the exactness probe reports
a mismatch, and the stream fingerprint."""
import hashlib

import numpy as np
import pytest

from exact_speculative_decoding_amd.loop import decode, rows_after_probe, token_sha


def _scripted(truth):
    """A verify pass that samples the true stream: row r at slot pos samples
    truth[pos + r - pos0] (the token after its input); commits by the accept rule."""
    calls = []

    def fn(tokens, pos):
        calls.append((pos, list(tokens)))
        R = len(tokens)
        sampled = [truth[pos - 100 + r] for r in range(R)]
        a = 0
        while a < R - 1 and tokens[a + 1] == sampled[a]:
            a += 1
        return sampled, min(a + 1, R)
    return fn, calls


def test_decode_commits_the_true_stream_with_any_drafter():
    rng = np.random.default_rng(0)
    truth = [int(t) for t in rng.integers(0, 50, 64)]
    for R, drafter in ((1, lambda p, c: []), (4, lambda p, c: [truth[p - 101 + i] for i in range(c)]),
                       (5, lambda p, c: [(truth[p - 101 + i] + 1) % 50 for i in range(c)])):
        fn, calls = _scripted(truth)
        out, rounds = decode(fn, 7, 100, 40, R, drafter)
        assert out == truth[:40]
        # every round starts at the slot after the previous round's commits
        slot, done = 100, 0
        for pos, tokens in calls:
            assert pos == slot and tokens[0] == (7 if done == 0 else truth[done - 1])
            _, n = fn(tokens, pos)  # the same pass again: its commit count
            calls.pop()
            slot, done = slot + n, done + n
        assert done == 40 and rounds == len(calls)


def test_probe_mismatch_falls_back_to_one_row():
    asked = []

    def exact(R):
        asked.append(R)
        return 0

    def broken(R):
        asked.append(R)
        return 3

    assert rows_after_probe(exact, 8) == 8
    assert rows_after_probe(broken, 8) == 1
    assert rows_after_probe(broken, 1) == 1
    assert asked == [8, 8]  # R = 1 needs no probe
    # a decode at the probed width: serial rounds when the probe fails
    rng = np.random.default_rng(1)
    truth = [int(t) for t in rng.integers(0, 50, 64)]
    good = lambda p, c: [truth[p - 101 + i] for i in range(c)]
    fn, calls = _scripted(truth)
    out, rounds = decode(fn, 7, 100, 30, rows_after_probe(broken, 8), good)
    assert out == truth[:30] and rounds == 30 and all(len(t) == 1 for _, t in calls)
    fn, calls = _scripted(truth)
    out, rounds = decode(fn, 7, 100, 30, rows_after_probe(exact, 8), good)
    assert out == truth[:30] and rounds == 4


def test_token_sha_is_sha256_of_int32_ids():
    toks = [0, 1, 151935, 2 ** 31 - 1]
    raw = b"".join(int(t).to_bytes(4, "little", signed=True) for t in toks)
    assert token_sha(toks) == hashlib.sha256(raw).hexdigest()
    assert token_sha(np.array(toks, np.int32)) == token_sha(toks)
    assert token_sha([1, 2]) != token_sha([2, 1])


def _scripted_chain(truth, proposer, cost, clock):
    """A verify pass over the true stream (as _scripted) that also proposes the
    next drafts with proposer(out) and advances a fake clock by cost(R)."""
    def fn(tokens, pos, out=None):
        R = len(tokens)
        sampled = [truth[pos - 100 + r] for r in range(R)]
        a = 0
        while a < R - 1 and tokens[a + 1] == sampled[a]:
            a += 1
        n = min(a + 1, R)
        clock[0] += cost(R)
        committed = (out or []) + sampled[:n]
        return sampled, n, proposer(committed, pos + n)
    return fn


def test_chained_decode_commits_the_true_stream():
    rng = np.random.default_rng(3)
    truth = [int(t) for t in rng.integers(0, 50, 80)]
    clock = [0.0]
    from exact_speculative_decoding_amd.loop import decode_chained
    # drafts: the next 3 true tokens (all accepted), or wrong ones (none)
    good = _scripted_chain(truth, lambda c, p: truth[p - 100:p - 97], lambda R: 1.0, clock)
    out, rounds = decode_chained(lambda t, p: good(t, p), 7, 100, 40)
    assert out == truth[:40] and rounds == 11  # 1, then 4 a round (9 rounds), then the last 3
    bad = _scripted_chain(truth, lambda c, p: [(t + 1) % 50 for t in truth[p - 100:p - 97]], lambda R: 1.0, clock)
    out, rounds = decode_chained(lambda t, p: bad(t, p), 7, 100, 40)
    assert out == truth[:40] and rounds == 40


def test_adaptive_choice_keeps_the_faster_drafter():
    from exact_speculative_decoding_amd.loop import decode_adaptive
    rng = np.random.default_rng(4)
    truth = [int(t) for t in rng.integers(0, 50, 200)]
    clock = [0.0]
    tick = lambda: clock[0]
    # "head": always right, 3 drafts, 2.0 time units a round (its probe: 1
    # token, then 4 a round: 13 in 8 units); "cheap": always wrong, 0.4 a
    # round (1 token each: 2.5 a unit) -- cheap commits more per unit of time
    head = _scripted_chain(truth, lambda c, p: truth[p - 100:p - 97], lambda R: 2.0, clock)
    cheap = _scripted_chain(truth, lambda c, p: [-1], lambda R: 0.4, clock)
    out, rounds, best, rate = decode_adaptive([("head", head), ("cheap", cheap)], 7, 100, 120, 4, tick)
    assert out == truth[:120]
    # head: its first round has no drafts (1 token), then 4 a round
    assert rate["head"] == pytest.approx(13 / 8.0) and rate["cheap"] == pytest.approx(1 / 0.4)
    assert best == "cheap"
    clock[0] = 0.0
    slow_cheap = _scripted_chain(truth, lambda c, p: [-1], lambda R: 1.5, clock)
    out, rounds, best, rate = decode_adaptive([("cheap", slow_cheap), ("head", head)], 7, 100, 120, 4, tick)
    assert out == truth[:120] and best == "head"


def test_lookup_drafts():
    from exact_speculative_decoding_amd.loop import lookup_drafts
    h = [5, 1, 2, 3, 9, 1, 2, 7, 1, 2]
    assert lookup_drafts(h, 3) == [7, 1, 2]   # last bigram (1, 2) most recently followed by 7
    assert lookup_drafts([4, 8, 4], 2) == [8, 4]
    assert lookup_drafts([1, 2, 3], 2) == []
