"""Seeded synthetic inputs for the verify-pass workloads.

This module only draws random numbers and encodes them into the storage
formats the library takes (bf16 / fp16 bit patterns, packed 4-bit weights).  It
holds none of the method's arithmetic, and it is the only code that both the
CPU oracle's tests and the GPU path consume.

Workloads (all draws from numpy's PCG64 `default_rng(seed)`):
  tiny      one W4 linear K=256 -> N=512, G=64, 4 lanes, sampler over V=512
  mlp       dense 27B-class MLP slice: gate/up 5120 -> 17408, down 17408 -> 5120, G=64
  lm_head   W4 5120 -> 151936, G=64, 64 hidden rows
  moe       hidden 2048, 128 experts, top-8, expert intermediate 768, G=32
  decoder   8-layer toy decoder (hidden 2048, 16 q / 4 kv heads, head dim 128,
            MLP 6144, vocab 32768, G=64)

Weight recipe: every 4-bit code is uniform on 0..15 (a uniform random byte is
two independent uniform nibbles), scale ~ U(0.01, 0.05) and bias ~ N(0, 0.1)
per group, both rounded to fp16; activations ~ N(0, 1) rounded to bf16.
"""
import numpy as np


def rng(seed):
    return np.random.default_rng(seed)


def bf16_bits(a):
    """Round float values to bf16 (nearest-even) and return the uint16 bits."""
    f = np.ascontiguousarray(a, dtype=np.float32)
    u = f.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + lsb) >> 16).astype(np.uint16)
    nan = np.isnan(f)
    if nan.any():
        r[nan] = 0x7FC0
    return r.reshape(np.shape(a))


def fp16_bits(a):
    """Round to IEEE binary16 (nearest-even, numpy) and return the uint16 bits."""
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64).astype(np.float16)).view(np.uint16)


def bf16_values(bits):
    """bf16 bits -> float32 values (for building test inputs only)."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


def w4_matrix(g, N, K, G):
    """Random packed 4-bit weights q [N][K/2] u8, scale/bias [N][K/G] fp16 bits."""
    assert K % G == 0 and K % 2 == 0
    q = g.integers(0, 256, size=(N, K // 2), dtype=np.uint8)
    s = fp16_bits(g.uniform(0.01, 0.05, size=(N, K // G)))
    b = fp16_bits(g.normal(0.0, 0.1, size=(N, K // G)))
    return q, s, b


def activations(g, R, K):
    return bf16_bits(g.standard_normal((R, K), dtype=np.float32))


# ---------------------------------------------------------------------------
# Workloads.
# ---------------------------------------------------------------------------

def tiny(seed=1001):
    """One W4 linear K=256 -> N=512 (G=64) on 4 lanes, and the sampler setting
    T=0.8, top-k 20, top-p 0.95, seed 42 over V=512."""
    g = rng(seed)
    q, s, b = w4_matrix(g, 512, 256, 64)
    x = activations(g, 4, 256)
    return dict(K=256, N=512, G=64, q=q, s=s, b=b, x=x,
                T=0.8, top_k=20, top_p=0.95, seed=42)


def mlp(seed=1002, H=5120, I=17408, G=64, R=16):
    g = rng(seed)
    gate = w4_matrix(g, I, H, G)
    up = w4_matrix(g, I, H, G)
    down = w4_matrix(g, H, I, G)
    x = activations(g, R, H)
    return dict(H=H, I=I, G=G, gate=gate, up=up, down=down, x=x)


def lm_head(seed=1003, K=5120, V=151936, G=64, rows=64):
    g = rng(seed)
    w = w4_matrix(g, V, K, G)
    h = activations(g, rows, K)
    return dict(K=K, V=V, G=G, w=w, h=h)


def moe(seed=1004, H=2048, I=768, E=128, top=8, G=32, R=16):
    g = rng(seed)
    gate = w4_matrix(g, E * I, H, G)
    up = w4_matrix(g, E * I, H, G)
    down = w4_matrix(g, E * H, I, G)
    stack = lambda w, rows: (w[0].reshape(E, rows, -1), w[1].reshape(E, rows, -1),
                             w[2].reshape(E, rows, -1))
    x = activations(g, R, H)
    rho = g.standard_normal((R, E), dtype=np.float32)
    return dict(H=H, I=I, E=E, top=top, G=G, gate=stack(gate, I), up=stack(up, I),
                down=stack(down, H), x=x, rho=rho)


def logits(g, R, V, scale=4.0):
    """Synthetic fp32 logit rows for sampler tests: N(0, scale^2)."""
    return (g.standard_normal((R, V)) * scale).astype(np.float32)


def draft_coins(seed, n, p):
    """Pre-drawn drafter decisions: accept-coin per slot with probability p, and a
    random offset 1..V-1 used to make a guaranteed-wrong guess."""
    g = rng(seed)
    return g.random(n) < p, g.integers(1, 1 << 30, size=n)


def decoder(seed=1005, layers=8, hidden=2048, heads=16, kv_heads=4, head_dim=128, inter=6144,
            vocab=32768, G=64, C=4096, prefill=None, rope_base=1e6, eps=1e-6):
    """Random-init decoder in standard layouts (the weight keys of the oracle's
    decoder), plus K/V caches [layers][kv_heads][C][head_dim] fp16 whose first
    `prefill` slots (default C - 512) hold N(0, 1) entries, the same bytes on
    every run.  RMSNorm gains are drawn from U(0.8, 1.2) rather than set to 1,
    so that a gain applied to the wrong element is visible."""
    g = rng(seed)
    nqkv, dq = (heads + 2 * kv_heads) * head_dim, heads * head_dim

    def stack(N, K):
        parts = [w4_matrix(g, N, K, G) for _ in range(layers)]
        return tuple(np.stack([p[i] for p in parts]) for i in range(3))

    w = {"embed": bf16_bits(g.standard_normal((vocab, hidden), dtype=np.float32)),
         "attn_norm": g.uniform(0.8, 1.2, (layers, hidden)).astype(np.float32),
         "mlp_norm": g.uniform(0.8, 1.2, (layers, hidden)).astype(np.float32),
         "final_norm": g.uniform(0.8, 1.2, hidden).astype(np.float32)}
    for name, (N, K) in (("qkv", (nqkv, hidden)), ("o", (hidden, dq)), ("gate", (inter, hidden)),
                         ("up", (inter, hidden)), ("down", (hidden, inter))):
        w[name + "_q"], w[name + "_s"], w[name + "_b"] = stack(N, K)
    w["lm_q"], w["lm_s"], w["lm_b"] = w4_matrix(g, vocab, hidden, G)
    prefill = C - 512 if prefill is None else prefill
    kc = np.zeros((layers, kv_heads, C, head_dim), np.uint16)
    vc = np.zeros((layers, kv_heads, C, head_dim), np.uint16)
    for l in range(layers):
        kc[l, :, :prefill] = fp16_bits(g.standard_normal((kv_heads, prefill, head_dim), dtype=np.float32))
        vc[l, :, :prefill] = fp16_bits(g.standard_normal((kv_heads, prefill, head_dim), dtype=np.float32))
    cfg = dict(layers=layers, hidden=hidden, heads=heads, kv_heads=kv_heads, head_dim=head_dim,
               inter=inter, vocab=vocab, G=G, rope_base=rope_base, eps=eps, C=C, prefill=prefill)
    first = int(g.integers(0, vocab))
    return dict(cfg=cfg, w=w, kc=kc, vc=vc, first_token=first)


def tiny_decoder(seed=1006, **kw):
    """A 2-layer decoder small enough for the oracle's exhaustive checks."""
    a = dict(layers=2, hidden=256, heads=2, kv_heads=1, head_dim=128, inter=384, vocab=512, G=64,
             C=64, prefill=8)
    a.update(kw)
    return decoder(seed, **a)


def transcript_drafter(transcript, pos_first, p, seed, V):
    """Drafts that equal a known serial transcript with probability p per
    position (pre-drawn coins keyed by position), else a token that is
    certainly wrong.  transcript[i] is the token at position pos_first + i."""
    n = len(transcript)
    coin, off = draft_coins(seed, n + 1, p)

    def draft(position, count):
        out = []
        for q in range(position, position + count):
            i = q - pos_first
            t = int(transcript[i]) if 0 <= i < n else 0
            out.append(t if (0 <= i < n and coin[i]) else (t + 1 + int(off[max(i, 0) % (n + 1)]) % (V - 1)) % V)
        return out
    return draft


def random_drafter(seed, V):
    """Drafts drawn uniformly over the vocabulary, keyed by position."""
    def draft(position, count):
        return [int(rng((seed, q)).integers(0, V)) for q in range(position, position + count)]
    return draft


def draft_head(seed, hidden, G):
    """W4 weights of a random-init MTP-style draft head (hidden x hidden), in
    the cfg-2 distributions (standard layout q, s, b)."""
    return w4_matrix(rng(seed), hidden, hidden, G)



def nvfp4_matrix(g, N, K, s_lo=0.002, s_hi=0.02):
    """An NVFP4-style N x K matrix in standard layout: q [N][K/2] (FP4 E2M1
    codes uniform over all 16, low nibble = even k), s [N][K/16] FP8 E4M3 block
    scales ~ U(s_lo, s_hi) rounded to nearest E4M3, and a tensor scale."""
    import torch
    codes = g.integers(0, 16, (N, K), dtype=np.uint8)
    q = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    sv = g.uniform(s_lo, s_hi, (N, K // 16)).astype(np.float32)
    s = torch.from_numpy(sv).to(torch.float8_e4m3fn).view(torch.uint8).numpy().copy()
    s_t = float(np.float32(g.uniform(0.5, 2.0)))
    return q, s, s_t
