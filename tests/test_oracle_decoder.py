"""Pins for the oracle's decoder step (oracle/decoder.c), each against something
other than the oracle's own formula:

* RMSNorm: a constant vector normalises to sign * gain exactly; scaling the
  input by a power of two changes no bit; with unit gains the output's mean
  square is 1 up to bf16 rounding.
* rotary positions: position 0 is the identity; a unit vector e_i turns in the
  (i, i + d/2) plane by p * theta_i, with theta_0 = 1 rad and theta_i =
  base^(-2i/d); norms are kept; the dot product of a rotated query and key
  depends only on the difference of their positions.
* attention: one slot returns that slot's value exactly; equal keys average
  the values; permuting the slots (keys and values together) changes nothing,
  permuting values alone does; two slots follow the logistic closed form,
  which fixes the 1/sqrt(d) scale.
* decoder step, special cases that reduce it to already-pinned pieces: with
  every layer's weights zero it is final norm + LM head of the embedding row;
  at position 0 with the MLP weights zero, each query head's attention output
  is its key/value head's value (GQA mapping), and the step is the o
  projection's residual update; the K/V slot written is the rotated key and
  the value in fp16.
* drafted decoding (rounds of R rows, each row one oracle step) commits the
  same tokens as serial decoding, with transcript and random drafters.
"""
import numpy as np
import pytest
from scipy.special import expit

import oracle
import synthetic as syn


def _f16(bits):
    return np.asarray(bits, np.uint16).view(np.float16).astype(np.float64)


# --- RMSNorm -----------------------------------------------------------------

def test_rmsnorm_constant_vector_and_gains():
    g = np.random.default_rng(1)
    gain = syn.bf16_values(syn.bf16_bits(g.uniform(0.5, 2.0, 64).astype(np.float32)))
    for c in (3.0, -0.125, 1e-3):
        out = oracle.rmsnorm_bf16(np.full(64, c, np.float32), gain, 0.0)
        assert np.array_equal(out, syn.bf16_bits(np.sign(c) * gain))


def test_rmsnorm_scale_invariance_and_unit_rms():
    g = np.random.default_rng(2)
    x = g.standard_normal(2048).astype(np.float32) * 7.0
    ones = np.ones(2048, np.float32)
    a = oracle.rmsnorm_bf16(x, ones, 0.0)
    for k in (-3, 5):
        assert np.array_equal(a, oracle.rmsnorm_bf16(x * np.float32(2.0 ** k), ones, 0.0))
    v = syn.bf16_values(a).astype(np.float64)
    assert abs(np.mean(v * v) - 1.0) < 4e-3  # bf16 rounding only
    gain = g.uniform(0.8, 1.2, 2048).astype(np.float32)
    b = syn.bf16_values(oracle.rmsnorm_bf16(x, gain, 0.0)).astype(np.float64)
    assert np.allclose(b, v * gain, rtol=2 ** -7, atol=0)


# --- rotary positions ---------------------------------------------------------

def test_rope_position_zero_is_identity():
    v = np.random.default_rng(3).standard_normal(128).astype(np.float32)
    assert np.array_equal(oracle.rope(v, 0, 1e6), v)


@pytest.mark.parametrize("i", [0, 1, 17, 63])
@pytest.mark.parametrize("p", [1, 5, 4095, 32767])
def test_rope_unit_vector_turns_in_its_plane(i, p):
    d, base = 128, 1e6
    e = np.zeros(d, np.float32)
    e[i] = 1.0
    out = oracle.rope(e, p, base).astype(np.float64)
    theta = 1.0 if i == 0 else base ** (-2.0 * i / d)
    assert out[i] == pytest.approx(np.cos(p * theta), abs=1e-7)
    assert out[i + 64] == pytest.approx(np.sin(p * theta), abs=1e-7)
    rest = np.delete(out, [i, i + 64])
    assert not rest.any()


def test_rope_keeps_norms_and_is_relative():
    g = np.random.default_rng(4)
    q = g.standard_normal(128).astype(np.float32)
    k = g.standard_normal(128).astype(np.float32)
    for p in (3, 1000, 30000):
        assert np.linalg.norm(oracle.rope(q, p, 1e6)) == pytest.approx(np.linalg.norm(q), rel=1e-6)
    dots = [np.dot(oracle.rope(q, p + 7, 1e6).astype(np.float64), oracle.rope(k, p, 1e6))
            for p in (0, 11, 500, 20000)]
    assert np.allclose(dots, dots[0], rtol=0, atol=2e-4 * np.linalg.norm(q) * np.linalg.norm(k))


# --- attention ------------------------------------------------------------------

def _kv(g, n, d=128):
    return (syn.fp16_bits(g.standard_normal((n, d))), syn.fp16_bits(g.standard_normal((n, d))))


def test_attention_single_slot_returns_its_value():
    g = np.random.default_rng(5)
    K, V = _kv(g, 1)
    q = g.standard_normal(128).astype(np.float32) * 30
    assert np.array_equal(oracle.attend(q, K, V), _f16(V[0]))


def test_attention_equal_keys_average_values():
    g = np.random.default_rng(6)
    K, V = _kv(g, 9)
    K[:] = K[0]
    q = g.standard_normal(128).astype(np.float32)
    assert np.allclose(oracle.attend(q, K, V), _f16(V).mean(axis=0), rtol=0, atol=1e-14)


def test_attention_is_a_function_of_the_slot_set():
    g = np.random.default_rng(7)
    K, V = _kv(g, 33)
    q = g.standard_normal(128).astype(np.float32) * 0.2
    o = oracle.attend(q, K, V)
    perm = g.permutation(33)
    assert np.allclose(oracle.attend(q, K[perm], V[perm]), o, rtol=0, atol=1e-13)
    assert not np.allclose(oracle.attend(q, K, V[perm]), o, rtol=0, atol=1e-3)


def test_attention_two_slots_closed_form():
    g = np.random.default_rng(8)
    K, V = _kv(g, 2)
    q = g.standard_normal(128).astype(np.float32) * 0.3
    k = _f16(K)
    delta = (np.dot(q, k[0]) - np.dot(q, k[1])) / np.sqrt(128.0)
    w0 = expit(delta)
    expect = w0 * _f16(V[0]) + (1.0 - w0) * _f16(V[1])
    assert np.allclose(oracle.attend(q, K, V), expect, rtol=0, atol=1e-12)


# --- decoder step special cases ---------------------------------------------------

SAMPLING = (0.7, 20, 0.95, 42)


def _zeroed(d, names):
    w = dict(d["w"])
    for n in names:
        for part in ("_q", "_s", "_b"):
            w[n + part] = np.zeros_like(w[n + part])
    return w


def test_step_with_zero_layers_is_lm_head_of_embedding():
    d = syn.tiny_decoder()
    w = _zeroed(d, ["qkv", "o", "gate", "up", "down"])
    m = oracle.Decoder(d["cfg"], w, d["kc"], d["vc"])
    t, pos = 77, 8
    logits, tok, _ = m.step(t, pos, *SAMPLING)
    x = syn.bf16_values(w["embed"][t])
    n = oracle.rmsnorm_bf16(x, w["final_norm"], d["cfg"]["eps"])
    ref = oracle.w4_linear(n[None], w["lm_q"], w["lm_s"], w["lm_b"], d["cfg"]["G"], out_f32=True)[0]
    assert np.array_equal(logits.view(np.uint32), ref.view(np.uint32))
    assert tok == oracle.sample_row(ref, pos + 1, *SAMPLING).token


def test_step_at_position_zero_is_value_through_o_projection():
    d = syn.tiny_decoder(heads=4, kv_heads=2, hidden=512, layers=1)
    cfg, w0 = d["cfg"], d["w"]
    w = _zeroed(d, ["gate", "up", "down"])
    m = oracle.Decoder(cfg, w, d["kc"], d["vc"])
    t = 5
    logits, _, _ = m.step(t, 0, *SAMPLING)
    H, D, NH, NKV, G, eps = cfg["hidden"], cfg["head_dim"], cfg["heads"], cfg["kv_heads"], cfg["G"], cfg["eps"]
    x = syn.bf16_values(w0["embed"][t]).astype(np.float32)
    n = oracle.rmsnorm_bf16(x, w0["attn_norm"][0], eps)
    qkv = oracle.w4_linear(n[None], w0["qkv_q"][0], w0["qkv_s"][0], w0["qkv_b"][0], G, out_f32=True)[0]
    v = qkv[(NH + NKV) * D:].reshape(NKV, D)
    k = qkv[NH * D:(NH + NKV) * D].reshape(NKV, D)
    v16 = syn.fp16_bits(v)
    o = np.concatenate([syn.bf16_bits(_f16(v16[h // (NH // NKV)]).astype(np.float32)) for h in range(NH)])
    oo = oracle.w4_linear(o[None], w0["o_q"][0], w0["o_s"][0], w0["o_b"][0], G, out_f32=True)[0]
    x1 = (x.astype(np.float64) + oo.astype(np.float64)).astype(np.float32)
    nf = oracle.rmsnorm_bf16(x1, w0["final_norm"], eps)
    ref = oracle.w4_linear(nf[None], w0["lm_q"], w0["lm_s"], w0["lm_b"], G, out_f32=True)[0]
    assert np.array_equal(logits.view(np.uint32), ref.view(np.uint32))
    # slot 0 of the caches: the key turned by position 0 (unchanged) and the value, in fp16
    assert np.array_equal(m.kc[0, :, 0], syn.fp16_bits(k))
    assert np.array_equal(m.vc[0, :, 0], v16)


def test_cache_slot_holds_rotated_key():
    d = syn.tiny_decoder(layers=1)
    cfg, w = d["cfg"], d["w"]
    m = oracle.Decoder(cfg, w, d["kc"], d["vc"])
    t, pos = 9, 20
    m.step(t, pos, *SAMPLING)
    H, D, NH, G = cfg["hidden"], cfg["head_dim"], cfg["heads"], cfg["G"]
    n = oracle.rmsnorm_bf16(syn.bf16_values(w["embed"][t]), w["attn_norm"][0], cfg["eps"])
    qkv = oracle.w4_linear(n[None], w["qkv_q"][0], w["qkv_s"][0], w["qkv_b"][0], G, out_f32=True)[0]
    k = oracle.rope(qkv[NH * D:(NH + 1) * D], pos, cfg["rope_base"])
    assert np.array_equal(m.kc[0, 0, pos], syn.fp16_bits(k))
    assert not m.kc[0, 0, pos + 1].any()


# --- drafted == serial ---------------------------------------------------------------

def test_drafted_decoding_equals_serial():
    # the oracle's own round loop (one row at a time, accept rule, rejected
    # rows' cache slots put back) against its serial loop
    d = syn.tiny_decoder()
    cfg = d["cfg"]
    pos0, n = cfg["prefill"], 40
    serial = oracle.Decoder(cfg, d["w"], d["kc"], d["vc"])
    ref = oracle.serial_decode(serial, d["first_token"], pos0, n, SAMPLING)
    one = oracle.Decoder(cfg, d["w"], d["kc"], d["vc"])
    got1, rounds1 = oracle.drafted_decode(one, d["first_token"], pos0, n, 1, lambda p, c: [], SAMPLING)
    assert got1 == ref and rounds1 == n
    V = cfg["vocab"]
    for R, drafter, helps in ((4, syn.transcript_drafter(ref, pos0 + 1, 0.65, 5, V), True),
                              (3, syn.random_drafter(6, V), False),
                              (8, syn.transcript_drafter(ref, pos0 + 1, 0.9, 7, V), True)):
        m = oracle.Decoder(cfg, d["w"], d["kc"], d["vc"])
        got, rounds = oracle.drafted_decode(m, d["first_token"], pos0, n, R, drafter, SAMPLING)
        assert got == ref
        assert rounds < n if helps else rounds <= n
        # committed slots hold the serial bytes; stale slots were put back
        assert np.array_equal(m.kc, serial.kc)
        assert np.array_equal(m.vc, serial.vc)


def test_drafted_round_count_with_perfect_and_wrong_drafts():
    # a drafter that always proposes the serial tokens commits R tokens a
    # round; one that is always wrong commits one token a round
    d = syn.tiny_decoder()
    cfg = d["cfg"]
    pos0, n, V = cfg["prefill"], 24, cfg["vocab"]
    ref = oracle.serial_decode(oracle.Decoder(cfg, d["w"], d["kc"], d["vc"]), d["first_token"], pos0, n, SAMPLING)
    good = lambda p, c: [ref[p - pos0 - 1 + i] for i in range(c)]
    bad = lambda p, c: [(ref[p - pos0 - 1 + i] + 1) % V for i in range(c)]
    for R in (2, 4, 6):
        got, rounds = oracle.drafted_decode(oracle.Decoder(cfg, d["w"], d["kc"], d["vc"]), d["first_token"],
                                            pos0, n, R, good, SAMPLING)
        assert got == ref and rounds == -(-n // R)
        got, rounds = oracle.drafted_decode(oracle.Decoder(cfg, d["w"], d["kc"], d["vc"]), d["first_token"],
                                            pos0, n, R, bad, SAMPLING)
        assert got == ref and rounds == n


def test_cache_entries_saturate_at_the_fp16_limit():
    # values beyond the largest finite fp16 are stored as +-65504, never inf
    d = syn.tiny_decoder(layers=1)
    cfg, w = d["cfg"], dict(d["w"])
    NH, NKV, D = cfg["heads"], cfg["kv_heads"], cfg["head_dim"]
    b = np.array(w["qkv_b"], copy=True)
    rows = slice((NH + NKV) * D, (NH + 2 * NKV) * D)  # the value rows
    b[0, rows] = syn.fp16_bits(np.full(b[0, rows].shape, 30000.0))
    w["qkv_b"] = b
    m = oracle.Decoder(cfg, w, d["kc"], d["vc"])
    t, pos = 3, 5
    m.step(t, pos, *SAMPLING)
    n = oracle.rmsnorm_bf16(syn.bf16_values(w["embed"][t]), w["attn_norm"][0], cfg["eps"])
    qkv = oracle.w4_linear(n[None], w["qkv_q"][0], w["qkv_s"][0], b[0], cfg["G"], out_f32=True)[0]
    v = qkv[(NH + NKV) * D:].reshape(NKV, D)
    assert np.max(np.abs(v)) > 65520  # these would round to infinity
    stored = _f16(m.vc[0, :, pos])
    assert np.all(np.isfinite(stored))
    big = np.abs(v) > 65504
    assert np.array_equal(stored[big], np.sign(v[big]) * 65504.0)
    assert np.array_equal(m.vc[0, :, pos][~big], syn.fp16_bits(v[~big]))
