"""GPU parity of verify_step on the toy decoder.

* row exactness: every row of an R-row verify step (logits, sampled token,
  cache slot) is bit-identical to a one-row step at its position from the
  same cache;
* drafted decoding (rounds of R rows, transcript drafter at 65 % and a random
  drafter) commits the same tokens and cache bytes as serial decoding (R = 1);
* against the oracle, teacher-forced on the GPU's committed stream: logits
  within 2e-3 per row (max-norm relative), tokens identical except where the
  oracle's two best perturbed scores are within 1e-4 (counted, reported);
* edge cases: the last slots of the cache, R = 16, greedy decoding.
Sizes: a 2-layer decoder (hidden 256, cache 64), the 8-layer decoder (hidden
2048, 16/4 heads, MLP 6144, vocab 32768) with caches of 4096 and 32768 slots.
"""
import hashlib

import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from exact_speculative_decoding_amd.loop import decode
from helpers import NEAR_TIE, ROW_REL_TOL, host, row_rel_err

pytestmark = pytest.mark.gpu

SAMPLED = (0.7, 20, 0.95, 42)
GREEDY = (0.0, 1, 1.0, 0)
TOPP_ONLY = (0.8, 0, 0.9, 42)  # no top-k: top-p over the whole vocabulary


def _gpu_round(m, sampling, logits_log=None):
    def fn(tokens, pos0):
        t = torch.tensor(tokens, dtype=torch.int32, device="cuda")
        lg = None
        if logits_log is not None:
            lg = torch.empty((len(tokens), m.cfg["vocab"]), dtype=torch.float32, device="cuda")
        s, n = m.verify_step(t, pos0, *sampling, logits=lg)
        if logits_log is not None:
            logits_log.append((pos0, tokens, host(lg)))
        return host(s).tolist(), int(host(n)[0])
    return fn


def _fresh(d):
    return ev.load_decoder(d["cfg"], d["w"], d["kc"], d["vc"])


def _teacher_forced(d, stream, pos0, sampling, positions, gpu_logits=None):
    """Oracle steps over the committed stream (first token at slot pos0).  For
    each checked position returns (row error of the GPU logits if given, oracle
    token == GPU token, oracle gap)."""
    m = oracle.Decoder(d["cfg"], d["w"], d["kc"], d["vc"])
    inputs = [d["first_token"]] + stream[:-1]
    out = []
    for i, t in enumerate(inputs[:max(positions) + 1]):
        logits, tok, gap = m.step(t, pos0 + i, *sampling)
        if i in positions:
            err = None
            if gpu_logits is not None:
                err = float(row_rel_err(gpu_logits[i][None], logits[None])[0])
            out.append((err, tok == stream[i], gap))
    return out


def _check_stream(res):
    near = 0
    for err, same, gap in res:
        if err is not None:
            assert err <= ROW_REL_TOL, err
        if not same:
            assert gap < NEAR_TIE, gap
            near += 1
    return near


# --- small decoder -----------------------------------------------------------------

@pytest.fixture(scope="module")
def tiny():
    return syn.tiny_decoder()


def test_tiny_rows_bit_identical_to_single_row_steps(tiny):
    d, cfg = tiny, tiny["cfg"]
    pos0 = cfg["prefill"]
    m = _fresh(d)
    serial, _ = decode(_gpu_round(m, SAMPLED), d["first_token"], pos0, 12, 1, lambda p, c: [])
    kc0, vc0 = m.k_cache.clone(), m.v_cache.clone()
    for R in (16, 5, 2):
        base = pos0 + 12
        tokens = [serial[-1]] + [(serial[i % 12] * 7 + i) % cfg["vocab"] for i in range(R - 1)]
        m.k_cache.copy_(kc0)
        m.v_cache.copy_(vc0)
        V = cfg["vocab"]
        lg = torch.empty((R, V), dtype=torch.float32, device="cuda")
        s, _ = m.verify_step(torch.tensor(tokens, dtype=torch.int32, device="cuda"), base, *SAMPLED, logits=lg)
        many_l, many_s = host(lg), host(s)
        kcR, vcR = m.k_cache.clone(), m.v_cache.clone()
        m.k_cache.copy_(kc0)
        m.v_cache.copy_(vc0)
        for r, t in enumerate(tokens):
            l1 = torch.empty((1, V), dtype=torch.float32, device="cuda")
            s1, n1 = m.verify_step(torch.tensor([t], dtype=torch.int32, device="cuda"), base + r, *SAMPLED,
                                   logits=l1)
            assert np.array_equal(host(l1)[0].view(np.uint32), many_l[r].view(np.uint32)), (R, r)
            assert int(host(s1)[0]) == int(many_s[r]) and int(host(n1)[0]) == 1
        assert torch.equal(m.k_cache, kcR) and torch.equal(m.v_cache, vcR)


@pytest.mark.parametrize("sampling", [SAMPLED, GREEDY, TOPP_ONLY])
def test_tiny_drafted_equals_serial_and_matches_oracle(tiny, sampling):
    d, cfg = tiny, tiny["cfg"]
    pos0, n, V = cfg["prefill"], 40, cfg["vocab"]
    m = _fresh(d)
    log = []
    serial, rounds = decode(_gpu_round(m, sampling, log), d["first_token"], pos0, n, 1, lambda p, c: [])
    assert rounds == n
    kc_s, vc_s = host(m.k_cache), host(m.v_cache_standard())
    gpu_logits = [x[2][0] for x in log]
    res = _teacher_forced(d, serial, pos0, sampling, set(range(n)), gpu_logits)
    near = _check_stream(res)
    print(f"tiny decoder, T={sampling[0]}: {near} near-tie positions of {n}")
    for R, drafter in ((4, syn.transcript_drafter(serial, pos0 + 1, 0.65, 11, V)), (16, syn.random_drafter(12, V)),
                       (8, syn.transcript_drafter(serial, pos0 + 1, 0.9, 13, V))):
        m2 = _fresh(d)
        got, rounds = decode(_gpu_round(m2, sampling), d["first_token"], pos0, n, R, drafter)
        assert got == serial, R
        L = pos0 + n
        assert np.array_equal(host(m2.k_cache)[:, :, :L], kc_s[:, :, :L])
        assert np.array_equal(host(m2.v_cache_standard())[:, :, :L], vc_s[:, :, :L])


def test_tiny_graph_replay_equals_eager(tiny):
    """Every round of a drafted decode (R = 1, 4, 16 and the shorter last
    rounds) replayed from captured steps, with the eager first kernel, host
    read-backs and drafting between replays, gives the same sampled tokens,
    commit counts and caches as the same rounds launched kernel by kernel."""
    d, cfg = tiny, tiny["cfg"]
    pos0, n, V = cfg["prefill"], 30, cfg["vocab"]
    ref = decode(_gpu_round(_fresh(d), SAMPLED), d["first_token"], pos0, n, 1, lambda p, c: [])[0]
    for R, drafter in ((1, lambda p, c: []), (4, syn.transcript_drafter(ref, pos0 + 1, 0.65, 5, V)),
                       (16, syn.random_drafter(9, V))):
        runs = []
        for graphs in (False, True):
            m = _fresh(d)
            m.set_graphs(graphs)
            log = []

            def fn(tokens, p0):
                s, c = m.verify_step(torch.tensor(tokens, dtype=torch.int32, device="cuda"), p0, *SAMPLED)
                out = (host(s).tolist(), int(host(c)[0]))
                log.append((p0, tuple(tokens), tuple(out[0]), out[1]))
                return out

            got, _ = decode(fn, d["first_token"], pos0, n, R, drafter)
            runs.append((got, log, host(m.k_cache), host(m.v_cache)))
            del m
        (g0, l0, k0, v0), (g1, l1, k1, v1) = runs
        assert l1 == l0, R  # every round: position, tokens, sampled, commit count
        assert g1 == g0 == ref
        assert np.array_equal(k1, k0) and np.array_equal(v1, v0)


def test_tiny_host_round_helper_matches_verify_step(tiny):
    """verify_step_host (the native host round: tokens passed to the first
    kernel by value, one read-back of the sampled tokens and the commit
    count) drives the same rounds as verify_step."""
    d, cfg = tiny, tiny["cfg"]
    pos0, n, V = cfg["prefill"], 24, cfg["vocab"]
    ref = decode(_gpu_round(_fresh(d), SAMPLED), d["first_token"], pos0, n, 1, lambda p, c: [])[0]
    for R in (1, 4, 16):
        drafter = syn.transcript_drafter(ref, pos0 + 1, 0.65, 5, V)
        logs = []
        for use_host in (False, True):
            m = _fresh(d)
            log = []

            def fn(tokens, p0):
                if use_host:
                    out = m.verify_step_host(tokens, p0, *SAMPLED)
                else:
                    s, c = m.verify_step(torch.tensor(tokens, dtype=torch.int32, device="cuda"), p0, *SAMPLED)
                    out = (host(s).tolist(), int(host(c)[0]))
                log.append((p0, tuple(tokens), tuple(out[0]), out[1]))
                return out

            got, _ = decode(fn, d["first_token"], pos0, n, R, drafter)
            assert got == ref, R
            logs.append(log)
            del m
        assert logs[0] == logs[1], R


def test_tiny_decodes_to_the_last_slot(tiny):
    d, cfg = tiny, tiny["cfg"]
    pos0 = cfg["prefill"]
    n = cfg["C"] - pos0  # the last step's row sits in slot C - 1
    m = _fresh(d)
    serial, _ = decode(_gpu_round(m, SAMPLED), d["first_token"], pos0, n, 1, lambda p, c: [])
    m2 = _fresh(d)
    got, _ = decode(_gpu_round(m2, SAMPLED), d["first_token"], pos0, n, 6,
                    syn.transcript_drafter(serial, pos0 + 1, 0.65, 3, cfg["vocab"]))
    assert got == serial
    with pytest.raises(ev.EvError):
        m2.verify_step(torch.zeros(2, dtype=torch.int32, device="cuda"), cfg["C"] - 1, *SAMPLED)


@pytest.mark.parametrize("kw", [dict(heads=32, kv_heads=8), dict(hidden=2176, inter=256)])
def test_tiny_decoder_launch_shapes(kw):
    """Shapes whose W4 launches take the other forms: 32 query heads give an o
    projection of K = 4096 (32 chunks: the 16-wave K-parts workgroups);
    hidden 2176 (17 chunks) puts q|k|v and gate/up on the halved launches and
    the LM head on its own plan.  Drafted equals serial, and the oracle checks
    every position's logits and token."""
    d = syn.tiny_decoder(seed=1007, **kw)
    cfg = d["cfg"]
    pos0, n, V = cfg["prefill"], 16, cfg["vocab"]
    m = _fresh(d)
    log = []
    serial, _ = decode(_gpu_round(m, SAMPLED, log), d["first_token"], pos0, n, 1, lambda p, c: [])
    m2 = _fresh(d)
    got, _ = decode(_gpu_round(m2, SAMPLED), d["first_token"], pos0, n, 5,
                    syn.transcript_drafter(serial, pos0 + 1, 0.65, 4, V))
    assert got == serial
    L = pos0 + n
    assert torch.equal(m2.k_cache[:, :, :L], m.k_cache[:, :, :L])
    assert torch.equal(m2.v_cache_standard()[:, :, :L], m.v_cache_standard()[:, :, :L])
    res = _teacher_forced(d, serial, pos0, SAMPLED, set(range(n)), [x[2][0] for x in log])
    near = _check_stream(res)
    print(f"{kw}: max row err {max(r[0] for r in res):.3e}, {near} near ties")


# --- 8-layer decoder ------------------------------------------------------------------

def _full(C):
    return syn.decoder(C=C)


@pytest.mark.parametrize("C,n,sampling", [(4096, 96, SAMPLED), (32768, 24, SAMPLED), (4096, 48, GREEDY)])
def test_full_decoder_drafted_equals_serial_and_oracle(C, n, sampling):
    """The 8-layer decoder: serial decoding of n tokens; drafted decoding (8
    rows a round, drafts matching the serial transcript at 65 %) commits the
    same tokens and cache bytes; and the oracle, teacher-forced on the
    committed stream, checks the GPU's logits (per-row relative error <=
    2e-3) and token at every one of the n positions."""
    print(f"full decoder C={C} n={n} T={sampling[0]}", flush=True)
    d = _full(C)
    cfg = d["cfg"]
    pos0, V = cfg["prefill"], cfg["vocab"]
    m = _fresh(d)
    log = []
    serial, _ = decode(_gpu_round(m, sampling, log), d["first_token"], pos0, n, 1, lambda p, c: [])
    kc_s, vc_s = m.k_cache.clone(), m.v_cache_standard()
    del m
    m2 = _fresh(d)
    got, rounds = decode(_gpu_round(m2, sampling), d["first_token"], pos0, n, 8,
                         syn.transcript_drafter(serial, pos0 + 1, 0.65, 21, V))
    assert got == serial
    L = pos0 + n
    assert torch.equal(m2.k_cache[:, :, :L], kc_s[:, :, :L])
    assert torch.equal(m2.v_cache_standard()[:, :, :L], vc_s[:, :, :L])
    sha = hashlib.sha256(np.array(serial, np.int32).tobytes()).hexdigest()[:16]
    print(f"C={C}: {n} tokens in {rounds} rounds of 8 rows ({n / rounds:.2f} per round), sha256 {sha}")
    del m2
    gpu_logits = [x[2][0] for x in log]
    res = _teacher_forced(d, serial, pos0, sampling, set(range(n)), gpu_logits)
    assert len(res) == n
    near = _check_stream(res)
    print(f"C={C} T={sampling[0]}: oracle at all {n} positions: max row err "
          f"{max(r[0] for r in res):.3e}, {near} near ties (gap < 1e-4)")


def test_tiny_one_capture_serves_every_seed(tiny):
    """The captured step keeps no sampling parameter: 50 seeds (and greedy,
    and other temperatures and top-k / top-p) decoded through one handle
    capture nothing after the first rounds, and every round equals the same
    round launched kernel by kernel."""
    d, cfg = tiny, tiny["cfg"]
    pos0, n, V = cfg["prefill"], 12, cfg["vocab"]
    settings = [(0.7, 20, 0.95, s) for s in range(50)] + [GREEDY, (1.0, 5, 0.5, 7), (0.3, 64, 1.0, 8)]
    settings += [(0.8, 0, 0.9, s) for s in range(5)]  # top-p over the whole vocabulary: a second capture per R
    mg, me = _fresh(d), _fresh(d)
    me.set_graphs(False)
    kc0, vc0 = mg.k_cache.clone(), mg.v_cache.clone()
    for samp in settings:
        logs = []
        for m in (mg, me):
            m.k_cache.copy_(kc0)
            m.v_cache.copy_(vc0)
            log = []

            def fn(tokens, p0):
                out = m.verify_step_host(tokens, p0, *samp)
                log.append((p0, tuple(tokens), tuple(out[0]), out[1]))
                return out

            serial = decode(fn, d["first_token"], pos0, n, 1, lambda p, c: [])[0]
            decode(fn, d["first_token"], pos0, n, 4, syn.transcript_drafter(serial, pos0 + 1, 0.65, 5, V))
            logs.append(log)
        assert logs[0] == logs[1], samp
    # one capture per row count (R = 1..4, the rounds' widths) and sampler
    # kind (top-k candidates or whole-vocabulary top-p), none per setting
    captures, cached = mg.graph_stats()
    print(f"{len(settings)} sampling settings: {captures} captures")
    assert 1 <= captures <= 8 and cached == captures
    assert me.graph_stats() == (0, 0)


def test_probe_finds_row_passes_exact(tiny):
    """verify_probe on the live shapes: an R-row pass and the same rows one
    at a time agree word for word (logits, samples, cache entries), so the
    round loop keeps drafting; the slots it wrote are then rewritten by the
    round that starts there, which still equals serial decoding."""
    from exact_speculative_decoding_amd.loop import rows_after_probe
    d, cfg = tiny, tiny["cfg"]
    pos0, n, V = cfg["prefill"], 20, cfg["vocab"]
    ref = decode(_gpu_round(_fresh(d), SAMPLED), d["first_token"], pos0, n, 1, lambda p, c: [])[0]
    m = _fresh(d)
    for R in (2, 8, 16):
        toks = torch.tensor([d["first_token"]] + [(7 * i + 3) % V for i in range(R - 1)], dtype=torch.int32,
                            device="cuda")
        for samp in (SAMPLED, GREEDY):
            assert m.verify_probe(toks, pos0, *samp) == 0, (R, samp)
    R = rows_after_probe(lambda r: m.verify_probe(torch.tensor([d["first_token"]] * r, dtype=torch.int32,
                                                                device="cuda"), pos0, *SAMPLED), 8)
    assert R == 8
    got, _ = decode(_gpu_round(m, SAMPLED), d["first_token"], pos0, n, R,
                    syn.transcript_drafter(ref, pos0 + 1, 0.65, 5, V))
    assert got == ref


def test_probe_on_the_full_decoder():
    print("probe: full decoder C=4096 R=8", flush=True)
    d = _full(4096)
    cfg = d["cfg"]
    m = _fresh(d)
    toks = torch.tensor([d["first_token"]] + [(31 * i + 5) % cfg["vocab"] for i in range(7)], dtype=torch.int32,
                        device="cuda")
    assert m.verify_probe(toks, cfg["prefill"], *SAMPLED) == 0
    assert m.verify_probe(toks[:1].repeat(16).contiguous(), cfg["prefill"] + 9, *GREEDY) == 0
