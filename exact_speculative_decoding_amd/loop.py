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
