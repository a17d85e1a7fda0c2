"""Host side of drafted decoding: the round loop around a verify step.

A round at committed length L runs the verify pass on R rows whose inputs are
the last committed token (slot L - 1) and R - 1 drafts; it commits the accepted
drafts plus the verifier's token at the first mismatch (TensorFold README,
exactness paragraph: a draft survives exactly when it equals the serially
sampled token).  The next round starts from the last committed token at slot
L - 1 + n_commit; the cache slots the rejected rows wrote are overwritten then.
With R = 1 every round is one serial step.
"""


def decode(round_fn, first_token, pos0, n_tokens, R, drafter, on_round=None):
    """Commit `n_tokens` tokens after `first_token` (at slot `pos0`).

    round_fn(tokens, pos) -> (sampled, n_commit): one verify pass over the
    list `tokens` (input of slot pos + r in row r).
    drafter(position, count) -> `count` draft tokens for positions
    position .. position + count - 1.
    Returns the committed tokens and the number of rounds."""
    out = []
    last, pos, rounds = int(first_token), int(pos0), 0
    while len(out) < n_tokens:
        r = min(R, n_tokens - len(out))
        tokens = [last] + [int(t) for t in drafter(pos + 1, r - 1)]
        sampled, n_commit = round_fn(tokens, pos)
        committed = [int(t) for t in sampled[:n_commit]]
        out.extend(committed)
        last, pos, rounds = committed[-1], pos + n_commit, rounds + 1
        if on_round is not None:
            on_round(tokens, sampled, n_commit)
    return out, rounds


def rows_after_probe(probe, R):
    """The rows a round may use: R when probe(R), a count of differing words
    between an R-row pass and the same rows stepped one at a time, is 0; else
    1 (serial decoding, the same output, slower).  The TensorFold README's
    model notes: a model checks at load that drafted rows reproduce one-row
    decoding on the machine, and drafts only when they do."""
    if R <= 1:
        return 1
    return R if int(probe(R)) == 0 else 1


def token_sha(tokens):
    """sha256 (hex) of a committed token stream, the ids as little-endian
    int32: a fingerprint of one reply, equal for drafted and serial decoding
    of the same request (the blog's FAQ: the server reports a token hash per
    reply)."""
    import hashlib
    import struct
    return hashlib.sha256(struct.pack(f"<{len(tokens)}i", *[int(t) for t in tokens])).hexdigest()


def decode_chained(round_fn, first_token, pos0, n_tokens, drafts=None, on_round=None):
    """Drafted decoding where each round also proposes the next round's
    drafts (an MTP-style head run after the verify pass): round_fn(tokens,
    pos) -> (sampled, n_commit, next_drafts), tokens = [last committed] + the
    drafts the previous round proposed (none in the first round, unless given).
    Returns the committed tokens and the number of rounds."""
    out = []
    last, pos, rounds = int(first_token), int(pos0), 0
    drafts = list(drafts or [])
    while len(out) < n_tokens:
        room = n_tokens - len(out)
        tokens = [last] + [int(t) for t in drafts[:room - 1]]
        sampled, n_commit, drafts = round_fn(tokens, pos)
        committed = [int(t) for t in sampled[:n_commit]]
        out.extend(committed)
        last, pos, rounds = committed[-1], pos + n_commit, rounds + 1
        if on_round is not None:
            on_round(tokens, sampled, n_commit)
    return out, rounds


def lookup_drafts(history, k, ngram=2):
    """Prompt-lookup drafts: the k tokens that followed the most recent earlier
    occurrence of the history's last `ngram` tokens (then of its last token),
    or none.  Needs no model; exact decoding makes any proposal safe."""
    h = list(history)
    for n in range(min(ngram, len(h) - 1), 0, -1):
        tail = h[-n:]
        for s in range(len(h) - n - 1, -1, -1):
            if h[s:s + n] == tail:
                return h[s + n:s + n + k]
    return []


def decode_adaptive(candidates, first_token, pos0, n_tokens, probe_rounds=4, clock=None):
    """Drafted decoding that measures its drafters and keeps the fastest (the
    TensorFold README's DGX Spark notes: per request, the MTP head is measured
    against a draft model and whichever commits more tokens per millisecond is
    kept).  candidates: list of (name, round_fn) with round_fn(tokens, pos, out)
    -> (sampled, n_commit, next_drafts), `out` the tokens committed so far.
    Each candidate runs probe_rounds rounds in turn (starting with no drafts),
    then the one with the most committed tokens per second of wall time
    decodes the rest.  Returns (tokens, rounds, chosen name, {name: tok/s})."""
    import time
    clock = clock or time.perf_counter
    out = []
    last, pos, rounds = int(first_token), int(pos0), 0
    rate = {}

    def run(fn, max_rounds):
        nonlocal last, pos, rounds
        drafts, done = [], 0
        t0, c0 = clock(), len(out)
        while len(out) < n_tokens and done < max_rounds:
            room = n_tokens - len(out)
            tokens = [last] + [int(t) for t in drafts[:room - 1]]
            sampled, n_commit, drafts = fn(tokens, pos, out)
            committed = [int(t) for t in sampled[:n_commit]]
            out.extend(committed)
            last, pos, rounds, done = committed[-1], pos + n_commit, rounds + 1, done + 1
        dt = clock() - t0
        return (len(out) - c0) / dt if dt > 0 else float("inf")

    for name, fn in candidates:
        if len(out) >= n_tokens:
            break
        rate[name] = run(fn, probe_rounds)
    best = max(rate, key=rate.get) if rate else candidates[0][0]
    if len(out) < n_tokens:
        run(dict(candidates)[best], 1 << 62)
    return out, rounds, best, rate
