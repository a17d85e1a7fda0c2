"""The MTP-style draft chain (toy_decoder_draft) and the drafted round loops
on the GPU.

* Decoding with the head's drafts (decode_chained: each round verifies the
  drafts the previous round proposed) commits exactly the serial tokens, with
  the 30 % confidence stop and without it (min_conf 0: always max_drafts).
* The drafts against the oracle's chain (oracle.draft_chain, teacher-forced
  on the GPU's committed stream: the final-normed hidden row of each round's
  last committed token): equal tokens and equal kept counts, except where a
  draft's two best logits are within 1e-4 or its confidence within 1e-4 of
  the threshold (counted).
* decode_adaptive races the head against prompt-lookup drafts and plain
  serial rounds; whichever it keeps, the output equals serial decoding.
"""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from exact_speculative_decoding_amd.loop import decode, decode_adaptive, decode_chained, lookup_drafts
from helpers import host

pytestmark = pytest.mark.gpu

SAMPLED = (0.7, 20, 0.95, 42)


def _setup(d, seed=31):
    cfg = d["cfg"]
    m = ev.load_decoder(cfg, d["w"], d["kc"], d["vc"])
    q, s, b = syn.draft_head(seed, cfg["hidden"], cfg["G"])
    head = ev.w4_pack(*(torch.from_numpy(np.ascontiguousarray(a.view(np.int16) if a.dtype == np.uint16 else a)).cuda()
                        for a in (q, s, b)), cfg["G"])
    return m, head, (q, s, b)


def _serial(d, n):
    cfg = d["cfg"]
    m = ev.load_decoder(cfg, d["w"], d["kc"], d["vc"])
    return decode(lambda t, p: m.verify_step_host(t, p, *SAMPLED), d["first_token"], cfg["prefill"], n, 1,
                  lambda p, c: [])[0]


def _chain_rounds(m, head, d, n, max_drafts, min_conf):
    log = []

    def fn(tokens, pos):
        s, c, dr = m.verify_and_draft_host(tokens, pos, *SAMPLED, head, max_drafts, min_conf)
        log.append((pos, c, s[c - 1], dr))
        return s, c, dr
    out, rounds = decode_chained(fn, d["first_token"], d["cfg"]["prefill"], n)
    return out, rounds, log


def _oracle_check(d, wd, out, log, max_drafts, min_conf):
    cfg = d["cfg"]
    om = oracle.Decoder(cfg, d["w"], d["kc"], d["vc"])
    pos0 = cfg["prefill"]
    hidden = {}
    inputs = [d["first_token"]] + out[:-1]
    for i, t in enumerate(inputs):
        _, tok, _, h = om.step(t, pos0 + i, *SAMPLED, hidden=True)
        hidden[pos0 + i] = h
    checked = skipped = 0
    for pos, c, last, drafts in log:
        s = pos + c - 1
        if s not in hidden:
            continue
        kept, steps = oracle.draft_chain(cfg, d["w"], wd, hidden[s], last, max_drafts, min_conf)
        close = any(g < 1e-4 or abs(p - min_conf) < 1e-4 for _, p, g in steps)
        if close:
            skipped += 1
            continue
        assert drafts == kept, (pos, drafts, kept, steps)
        checked += 1
    return checked, skipped


@pytest.mark.parametrize("max_drafts,min_conf", [(3, 0.3), (6, 0.0), (3, 0.9), (4, 0.99)])
def test_tiny_chain_equals_serial_and_oracle(max_drafts, min_conf):
    d = syn.tiny_decoder()
    n = 40
    ref = _serial(d, n)
    m, head, wd = _setup(d)
    out, rounds, log = _chain_rounds(m, head, d, n, max_drafts, min_conf)
    assert out == ref
    nd = [len(x[3]) for x in log]
    if min_conf == 0.0:
        assert all(k == max_drafts for k in nd)
    if min_conf >= 0.9:
        assert min(nd) < max_drafts  # the confidence stop cut some chains short
    checked, skipped = _oracle_check(d, wd, out, log, max_drafts, min_conf)
    print(f"max_drafts {max_drafts}, min_conf {min_conf}: {rounds} rounds, drafts a round {np.mean(nd):.2f}; "
          f"oracle: {checked} rounds equal, {skipped} near a tie or the threshold")
    assert checked >= len(log) // 2


def test_full_decoder_chain_and_adaptive_choice():
    print("draft chain: full decoder C=4096", flush=True)
    d = syn.decoder(C=4096)
    cfg = d["cfg"]
    n = 48
    ref = _serial(d, n)
    m, head, wd = _setup(d)
    out, rounds, log = _chain_rounds(m, head, d, n, 3, 0.0)
    assert out == ref
    checked, skipped = _oracle_check(d, wd, out[:12], [x for x in log if x[0] + x[1] - 1 < cfg["prefill"] + 12], 3,
                                     0.0)
    print(f"full decoder: {rounds} rounds; oracle: {checked} rounds equal, {skipped} near a tie")
    # the race: head chain, prompt lookup, serial rounds
    m.k_cache.copy_(torch.from_numpy(d["kc"].view(np.int16)).cuda())
    m.v_cache.copy_(torch.from_numpy(np.ascontiguousarray(ev.v_cache_blocked(d["vc"])).view(np.int16)).cuda())
    hist = [d["first_token"]]

    def head_round(tokens, pos, done):
        return m.verify_and_draft_host(tokens, pos, *SAMPLED, head, 3, 0.3)

    def lookup_round(tokens, pos, done):
        s, c = m.verify_step_host(tokens, pos, *SAMPLED)
        return s, c, lookup_drafts([d["first_token"]] + done + s[:c], 3)

    def serial_round(tokens, pos, done):
        s, c = m.verify_step_host(tokens[:1], pos, *SAMPLED)
        return s, c, []

    out, rounds, best, rate = decode_adaptive([("mtp", head_round), ("lookup", lookup_round),
                                               ("serial", serial_round)], d["first_token"], cfg["prefill"], n, 4)
    assert out == ref
    print(f"adaptive: kept {best}; committed tok/s per drafter {({k: round(v) for k, v in rate.items()})}")
