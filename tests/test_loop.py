"""Host round loop (no GPU): the commit rule and next position on a scripted
verify pass, the fallback to one row a round when the exactness probe reports
a mismatch, and the stream fingerprint."""
import hashlib

import numpy as np

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
