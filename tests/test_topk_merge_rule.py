"""The selection rule of the vocab top-k kernel, emulated on the CPU: each of
four waves (64 lanes x 16 keys, every lane's keys sorted) takes its own top-kk
by rounds of a wave maximum over the lanes' heads, then each candidate's place
is its index in its own list plus the number of larger keys in the other three
lists.  For unique keys this gives exactly the chunk's top-kk in order, also
with many equal values (the id in the key breaks them) and with a partial last
chunk (key 0 = no logit).  The GPU parity tests check the kernel itself."""
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
