"""The selection rules of the sampler's kernels, emulated on the CPU.

* Rounds (the top-k kernel's fallback): each of four waves (64 lanes x 16
  keys, every lane's keys sorted) takes its own top-kk by rounds of a wave
  maximum over the lanes' heads, then each candidate's place is its index in
  its own list plus the number of larger keys in the other three lists.
* Bound and rank (the top-k kernel for kk > 2): t = the kk-th largest maximum
  of groups of 4 adjacent threads (2 when kk > 32); the keys >= t, in any
  order, are placed by the number of larger ones, unless more than 256 reach
  t.
* The merge kernel's bound: the kk-th largest of the first ceil(kk / nchunk)
  keys of every chunk list; the keys >= t are placed by rank.
For unique keys each gives exactly the top-kk in order, also with many equal
values (the id in the key breaks them) and with a partial last chunk (key 0 =
no logit).  The GPU parity tests check the kernels themselves."""
import numpy as np


def _select(thread_keys, kk):
    keys = -np.sort(-thread_keys, axis=1)  # each thread's 16 keys, descending
    lists = np.zeros((4, kk), np.int64)
    for w in range(4):
        lanes = keys[64 * w:64 * w + 64]
        at = np.zeros(64, int)
        for rnd in range(kk):
            heads = np.where(at < 16, lanes[np.arange(64), np.minimum(at, 15)], 0)
            m = heads.max()
            lists[w, rnd] = m
            if m != 0:
                assert (heads == m).sum() == 1
                at[int(np.argmax(heads == m))] += 1
    out = np.zeros(kk, np.int64)
    for v in range(4):
        for i in range(kk):
            e = lists[v, i]
            if e == 0:
                continue
            place = i + sum(int((lists[u] > e).sum()) for u in range(4) if u != v)
            if place < kk:
                out[place] = e
    return out


def test_wave_lists_and_counting_give_the_exact_top_k():
    rng = np.random.default_rng(5)
    for trial in range(60):
        kk = int(rng.integers(1, 65))
        nreal = int(rng.integers(1, 4097)) if trial % 3 == 0 else 4096
        vals = rng.integers(0, 50, size=4096) if trial % 2 else rng.integers(0, 1 << 20, size=4096)
        keys = ((vals.astype(np.int64) << 20) | (4095 - np.arange(4096))) + 1  # value desc, id asc
        keys[nreal:] = 0
        got = _select(keys.reshape(16, 256).T, kk)  # thread t holds logits i * 256 + t
        want = -np.sort(-keys)[:kk]
        assert np.array_equal(got, want), (trial, kk, nreal)


def _kth_nonzero(sample, kk):
    """The kk-th largest nonzero key of the sample, or 0 with fewer than kk."""
    nz = np.sort(sample[sample != 0])[::-1]
    return int(nz[kk - 1]) if len(nz) >= kk else 0


def _rank_place(cand, kk):
    out = np.zeros(kk, np.int64)
    for e in cand:
        rank = int((cand > e).sum())
        if rank < kk:
            out[rank] = e
    return out


def _chunk_bound_rank(thread_keys, kk):
    """None when the kernel falls back to rounds (more than 256 candidates).
    As the kernel: each thread's maximum, its keys >= t in load order (no sort)."""
    gs = 4 if kk <= 32 else 2
    t = _kth_nonzero(thread_keys.max(axis=1).reshape(-1, gs).max(axis=1), kk)
    cand = thread_keys[(thread_keys >= t) & (thread_keys != 0)]
    return None if len(cand) > 256 else _rank_place(cand, kk)


def _chunk_keys(rng, trial, nreal):
    vals = rng.integers(0, 50, size=4096) if trial % 2 else rng.integers(0, 1 << 20, size=4096)
    if trial % 5 == 4:  # values fall by one every four positions mod 256: the bound is loose
        vals = 1000 - (np.arange(4096) % 256) // 4
    keys = ((vals.astype(np.int64) << 20) | (4095 - np.arange(4096))) + 1
    keys[nreal:] = 0
    return keys


def test_chunk_bound_and_rank_give_the_exact_top_k():
    rng = np.random.default_rng(6)
    fallbacks = 0
    for trial in range(80):
        kk = int(rng.integers(3, 65))
        nreal = int(rng.integers(1, 4097)) if trial % 3 == 0 else 4096
        keys = _chunk_keys(rng, trial, nreal)
        got = _chunk_bound_rank(keys.reshape(16, 256).T, kk)
        want = -np.sort(-keys)[:kk]
        if got is None:  # the kernel selects in rounds
            fallbacks += 1
            got = _select(keys.reshape(16, 256).T, kk)
        assert np.array_equal(got, want), (trial, kk, nreal)
    assert 0 < fallbacks < 80


def test_merge_bound_and_rank_give_the_exact_top_k():
    rng = np.random.default_rng(7)
    for trial in range(80):
        kk = int(rng.integers(3, 65))
        nchunk = int(rng.integers(1, 65))
        vals = rng.integers(0, 1 << 20, size=(nchunk, 4096)) if trial % 2 else rng.integers(0, 30, size=(nchunk, 4096))
        ids = np.arange(nchunk * 4096).reshape(nchunk, 4096)
        keys = ((vals.astype(np.int64) << 24) | ((1 << 24) - 1 - ids)) + 1
        if trial % 4 == 3:  # a partial last chunk
            keys[-1, int(rng.integers(1, 4096)):] = 0
        lists = -np.sort(-keys, axis=1)[:, :kk]  # each chunk's top-kk (0 pads)
        ms = -(-kk // nchunk)
        t = _kth_nonzero(lists[:, :ms].ravel(), kk)
        cand = lists[(lists >= t) & (lists != 0)]
        want = -np.sort(-keys.ravel())[:kk]
        if len(cand) <= 256:
            assert np.array_equal(_rank_place(cand, kk), want), (trial, kk, nchunk)
        else:  # the merge rounds: the kk largest list keys in order
            assert np.array_equal(-np.sort(-lists.ravel())[:kk], want)
