"""numpy wrappers of oracle/decoder.c (TEST INFRASTRUCTURE): RMSNorm, rotary
positions, single-query attention, and the serial decoding step of the small
decoder.  Imported only through the `oracle` package."""
import ctypes as C

import numpy as np


def declare(L):
    u16, i32, i64, f32, f64 = C.c_uint16, C.c_int32, C.c_int64, C.c_float, C.c_double
    P = C.POINTER
    L.ov_rmsnorm_bf16.argtypes = [P(f32), i32, P(f32), f64, P(u16)]
    L.ov_rope.argtypes = [P(f32), i32, i64, f64]
    L.ov_attend.argtypes = [P(f32), P(u16), P(u16), i32, i32, P(f64)]
    L.ov_decoder_step.argtypes = [P(i32), P(f64), P(C.c_void_p), P(u16), P(u16), i32, i32, i64,
                                  f64, i32, f64, C.c_uint64, P(f32), P(i32), P(f64)]
    L.ov_decoder_step_h.argtypes = [P(i32), P(f64), P(C.c_void_p), P(u16), P(u16), i32, i32, i64,
                                    f64, i32, f64, C.c_uint64, P(f32), P(i32), P(f64), P(u16)]


def _lib():
    from . import lib
    return lib()


def _ptr(a, dt):
    from . import ptr
    return ptr(a, dt)


def rmsnorm_bf16(x, gain, eps):
    x = np.ascontiguousarray(x, np.float32)
    gain = np.ascontiguousarray(gain, np.float32)
    out = np.empty(x.shape, np.uint16)
    _lib().ov_rmsnorm_bf16(_ptr(x, np.float32), x.size, _ptr(gain, np.float32), float(eps),
                           _ptr(out, np.uint16))
    return out


def rope(v, pos, base):
    v = np.array(v, np.float32)
    _lib().ov_rope(_ptr(v, np.float32), v.size, int(pos), float(base))
    return v


def attend(q, K, V):
    q = np.ascontiguousarray(q, np.float32)
    K = np.ascontiguousarray(K, np.uint16)
    V = np.ascontiguousarray(V, np.uint16)
    n, d = K.shape
    o = np.empty(d, np.float64)
    _lib().ov_attend(_ptr(q, np.float32), _ptr(K, np.uint16), _ptr(V, np.uint16), n, d,
                     _ptr(o, np.float64))
    return o


# weight order of ov_decoder_step's pointer table
WEIGHT_KEYS = ["embed", "attn_norm", "mlp_norm", "final_norm",
               "qkv_q", "qkv_s", "qkv_b", "o_q", "o_s", "o_b",
               "gate_q", "gate_s", "gate_b", "up_q", "up_s", "up_b",
               "down_q", "down_s", "down_b", "lm_q", "lm_s", "lm_b"]
_DT = {"embed": np.uint16, "attn_norm": np.float32, "mlp_norm": np.float32,
       "final_norm": np.float32}


class Decoder:
    """The oracle decoder on a weight dict (standard layouts, see decoder.c)
    with its own copies of the K/V caches [L][kv_heads][C][d] fp16."""

    def __init__(self, cfg, weights, kc, vc):
        self.cfg = cfg
        self.ci = np.array([cfg["layers"], cfg["hidden"], cfg["heads"], cfg["kv_heads"],
                            cfg["head_dim"], cfg["inter"], cfg["vocab"], cfg["G"]], np.int32)
        self.cd = np.array([cfg["rope_base"], cfg["eps"]], np.float64)
        self.w = [np.ascontiguousarray(weights[k], _DT.get(k, np.uint8 if k.endswith("_q")
                                                           else np.uint16)) for k in WEIGHT_KEYS]
        self.tab = (C.c_void_p * len(self.w))(*[a.ctypes.data for a in self.w])
        self.kc = np.array(kc, np.uint16, copy=True)
        self.vc = np.array(vc, np.uint16, copy=True)
        self.C = self.kc.shape[2]

    def step(self, token, pos, T, top_k, top_p, seed, hidden=False):
        """Token at slot `pos` -> (logits of position pos + 1 [V] fp32, the token
        sampled there, its gap), and with hidden=True also the final-normed
        hidden row (the LM head's bf16 input).  Writes slot `pos` of the caches."""
        V = self.cfg["vocab"]
        logits = np.empty(V, np.float32)
        tok = np.zeros(1, np.int32)
        gap = np.zeros(1, np.float64)
        h = np.empty(self.cfg["hidden"], np.uint16)
        _lib().ov_decoder_step_h(_ptr(self.ci, np.int32), _ptr(self.cd, np.float64), self.tab,
                                 _ptr(self.kc, np.uint16), _ptr(self.vc, np.uint16), self.C,
                                 int(token), int(pos), float(T), int(top_k), float(top_p),
                                 int(seed) & ((1 << 64) - 1), _ptr(logits, np.float32),
                                 _ptr(tok, np.int32), _ptr(gap, np.float64), _ptr(h, np.uint16))
        if hidden:
            return logits, int(tok[0]), float(gap[0]), h
        return logits, int(tok[0]), float(gap[0])


def serial_decode(m, first_token, slot0, n, sampling):
    """Serial decoding on the oracle decoder `m`: `first_token` sits at slot
    `slot0`; each step feeds the last token at the next slot and keeps the
    token it samples.  Returns the n sampled tokens."""
    out, tok = [], int(first_token)
    for i in range(n):
        _, tok, _ = m.step(tok, slot0 + i, *sampling)
        out.append(tok)
    return out


def drafted_decode(m, first_token, slot0, n, R, drafter, sampling):
    """Drafted decoding on the oracle decoder, one row at a time (the accept
    rule of the TensorFold README's exactness paragraph: a draft is kept
    exactly when it equals the token sampled at its position).

    The stream s holds the committed tokens after `first_token`; with L tokens
    committed before a round (the last input at slot slot0 + L), the round's
    rows are the inputs [last, d_0, .., d_{W-2}] at slots slot0 + L + r, W =
    min(R, n - L) and drafter(position, count) giving the drafts for the
    positions after the last input.  Each row is one serial oracle step.  With
    a the number of leading drafts equal to the samples before them, the round
    keeps samples 0..min(a + 1, W) - 1, and the cache slots the rejected rows
    wrote are put back as they were before the round.  Returns (tokens,
    rounds)."""
    from . import accept
    s, rounds = [], 0
    last = int(first_token)
    while len(s) < n:
        L = len(s)
        W = min(R, n - L)
        base = slot0 + L
        drafts = [int(t) for t in drafter(base + 1, W - 1)]
        inputs = [last] + drafts
        kc0, vc0 = m.kc[:, :, base:base + W].copy(), m.vc[:, :, base:base + W].copy()
        samples = [m.step(t, base + r, *sampling)[1] for r, t in enumerate(inputs)]
        _, keep = accept(np.array(samples, np.int32), np.array(drafts, np.int32))
        m.kc[:, :, base + keep:base + W] = kc0[:, :, keep:]
        m.vc[:, :, base + keep:base + W] = vc0[:, :, keep:]
        s.extend(samples[:keep])
        last = samples[keep - 1]
        rounds += 1
    return s, rounds


def draft_chain(cfg, weights, w_draft, hidden, token, max_drafts, min_conf):
    """The MTP-style draft chain, one draft at a time, from the final-normed
    hidden row `hidden` (bf16 bits) of the last committed token `token`:
    a = bf16(h + embed[t]); z = W_draft a (W4, fp32 out); h = bf16(RMSNorm(z)
    * final_norm); logits = W_lm h; the draft is the argmax (lower id on
    ties) and its confidence the softmax probability 1 / sum_j exp(l_j - l_max)
    (fp64).  The chain stops at the first draft whose confidence is below
    min_conf.  Returns (drafts kept, every draft's (token, confidence, gap
    between the two best logits)) for all max_drafts steps."""
    from . import f64_to_bf16, w4_linear
    G, eps = cfg["G"], cfg["eps"]
    embed = np.asarray(weights["embed"], np.uint16)
    h, t = np.asarray(hidden, np.uint16), int(token)
    steps, kept, stopped = [], [], False
    for _ in range(max_drafts):
        hv = (np.asarray(h, np.uint32) << 16).view(np.float32).astype(np.float64)
        ev_ = (np.asarray(embed[t], np.uint32) << 16).view(np.float32).astype(np.float64)
        a = f64_to_bf16(hv + ev_)  # the exact sum, rounded once
        z = w4_linear(a[None], *w_draft, G, out_f32=True)[0]
        h = rmsnorm_bf16(z, weights["final_norm"], eps)
        logits = w4_linear(h[None], weights["lm_q"], weights["lm_s"], weights["lm_b"], G, out_f32=True)[0]
        l = logits.astype(np.float64)
        t = int(np.argmax(l))
        p = 1.0 / np.sum(np.exp(l - l[t]))
        top2 = np.sort(l)[-2:]
        steps.append((t, float(p), float(top2[1] - top2[0])))
        if not stopped and p >= min_conf:
            kept.append(t)
        else:
            stopped = True
    return kept, steps

