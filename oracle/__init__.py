"""CPU oracle for the exact drafted-decoding verify pass (TEST INFRASTRUCTURE).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It wraps oracle/liboracle.so (plain C, fp64, serial rows) with
numpy in and numpy out.  Nothing here touches the GPU or the HIP library.
"""
import ctypes as C
import os

import numpy as np

from . import build as _build

_HERE = os.path.dirname(os.path.abspath(__file__))
_lib = None


def lib():
    global _lib
    if _lib is None:
        path = _build.LIB
        srcs = [s for s in _build.SRC if os.path.exists(s)]
        if (not os.path.exists(path)) or any(
                os.path.getmtime(s) > os.path.getmtime(path) for s in srcs):
            _build.build()
        _lib = C.CDLL(path)
        _declare(_lib)
    return _lib


def _p(t):
    return C.POINTER(t)


class SampleOut(C.Structure):
    _fields_ = [("token", C.c_int32), ("gap", C.c_double), ("n_cand", C.c_int32),
                ("n_kept", C.c_int32), ("topp_edge", C.c_int32)]


def _declare(L):
    u8, u16, i32, i64, f32, f64 = (C.c_uint8, C.c_uint16, C.c_int32, C.c_int64,
                                   C.c_float, C.c_double)
    L.ov_bf16_to_f64.argtypes = [u16]
    L.ov_bf16_to_f64.restype = f64
    L.ov_f16_to_f64.argtypes = [u16]
    L.ov_f16_to_f64.restype = f64
    L.ov_f64_to_bf16.argtypes = [f64]
    L.ov_f64_to_bf16.restype = u16
    L.ov_f64_to_f16.argtypes = [f64]
    L.ov_f64_to_f16.restype = u16
    L.ov_mix64.argtypes = [C.c_uint64]
    L.ov_mix64.restype = C.c_uint64
    L.ov_noise_hash.argtypes = [C.c_uint64, i64, i32]
    L.ov_noise_hash.restype = C.c_uint64
    L.ov_uniform.argtypes = [C.c_uint64]
    L.ov_uniform.restype = f64
    L.ov_gumbel.argtypes = [C.c_uint64]
    L.ov_gumbel.restype = f64
    L.ov_num_threads.restype = C.c_int
    L.ov_set_num_threads.argtypes = [C.c_int]
    L.ov_set_num_threads.restype = None
    L.ov_silu.argtypes = [f64]
    L.ov_silu.restype = f64
    L.ov_w4_linear.argtypes = [_p(u16), i32, i32, _p(u8), _p(u16), _p(u16), i32, i32, _p(f64)]
    L.ov_w4_linear_f32.argtypes = [_p(u16), i32, i32, _p(u8), _p(u16), _p(u16), i32, i32, _p(f32)]
    L.ov_w4_linear_fp32.argtypes = [_p(u16), i32, i32, _p(u8), _p(u16), _p(u16), i32, i32, _p(f32)]
    L.ov_e2m1_to_f64.argtypes = [i32]
    L.ov_e2m1_to_f64.restype = f64
    L.ov_e4m3_to_f64.argtypes = [u8]
    L.ov_e4m3_to_f64.restype = f64
    L.ov_nvfp4_linear_f32.argtypes = [_p(u16), i32, i32, _p(u8), _p(u8), f32, i32, _p(f32)]
    L.ov_silu_mul_bf16.argtypes = [_p(f32), _p(f32), C.c_size_t, _p(u16)]
    L.ov_mlp.argtypes = [_p(u16), i32, i32, i32, i32,
                         _p(u8), _p(u16), _p(u16), _p(u8), _p(u16), _p(u16),
                         _p(u8), _p(u16), _p(u16), _p(f32), _p(f32), _p(f32), _p(u16)]
    L.ov_topk.argtypes = [_p(f32), i32, i32, _p(i32)]
    L.ov_topk.restype = i32
    L.ov_sample_from_candidates.argtypes = [_p(f32), _p(i32), i32, i64, f64, f64,
                                            C.c_uint64, _p(SampleOut)]
    L.ov_sample_row.argtypes = [_p(f32), i32, i64, f64, i32, f64, C.c_uint64, _p(SampleOut)]
    L.ov_sample_rows.argtypes = [_p(f32), i32, i32, _p(i64), f64, i32, f64, C.c_uint64,
                                 _p(i32), _p(f64), _p(i32), _p(i32)]
    L.ov_sample_many.argtypes = [_p(f32), i32, i32, _p(i64), _p(C.c_uint64), f64, i32, f64,
                                 _p(i32)]
    L.ov_accept.argtypes = [_p(i32), i32, _p(i32), i32, _p(i32), _p(i32)]
    L.ov_moe_route.argtypes = [_p(f32), i32, i32, _p(i32), _p(f64)]
    L.ov_moe.argtypes = [_p(u16), _p(f32), i32, i32, i32, i32, i32, i32,
                         _p(u8), _p(u16), _p(u16), _p(u8), _p(u16), _p(u16),
                         _p(u8), _p(u16), _p(u16), _p(f32), _p(i32), _p(f64)]
    if hasattr(L, "ov_decoder_step"):
        _declare_decoder(L)


def _declare_decoder(L):
    from . import decoder as _dec
    _dec.declare(L)


_CT = {np.uint8: C.c_uint8, np.uint16: C.c_uint16, np.int32: C.c_int32,
       np.int64: C.c_int64, np.float32: C.c_float, np.float64: C.c_double}


def ptr(a, dtype):
    """Pointer to a C-contiguous numpy array of exactly `dtype` (checked)."""
    if a is None:
        return None
    assert isinstance(a, np.ndarray) and a.dtype == np.dtype(dtype), (a.dtype, dtype)
    assert a.flags["C_CONTIGUOUS"]
    return a.ctypes.data_as(C.POINTER(_CT[np.dtype(dtype).type]))


def _c(a, dtype):
    return np.ascontiguousarray(a, dtype=dtype)


# --- number formats --------------------------------------------------------

def bf16_to_f64(bits):
    L = lib()
    return np.array([L.ov_bf16_to_f64(int(b)) for b in np.ravel(bits)]).reshape(np.shape(bits))


def f16_to_f64(bits):
    L = lib()
    return np.array([L.ov_f16_to_f64(int(b)) for b in np.ravel(bits)]).reshape(np.shape(bits))


def f64_to_bf16(v):
    L = lib()
    return np.array([L.ov_f64_to_bf16(float(x)) for x in np.ravel(v)],
                    dtype=np.uint16).reshape(np.shape(v))


def f64_to_f16(v):
    L = lib()
    return np.array([L.ov_f64_to_f16(float(x)) for x in np.ravel(v)],
                    dtype=np.uint16).reshape(np.shape(v))


# --- keyed noise -------------------------------------------------------------

def mix64(z):
    return int(lib().ov_mix64(z))


def noise_hash(seed, pos, tok):
    return int(lib().ov_noise_hash(seed, pos, tok))


def uniform(h):
    return float(lib().ov_uniform(h))


def gumbel(h):
    return float(lib().ov_gumbel(h))


def num_threads():
    return int(lib().ov_num_threads())


def set_num_threads(n):
    """OpenMP threads of the column loops (timing only: values do not change)."""
    lib().ov_set_num_threads(int(n))


def silu(v):
    return float(lib().ov_silu(v))


# --- W4 linear, MLP ----------------------------------------------------------

def w4_linear(x, q, s, b, G, out_f32=False):
    """x [R][K] bf16 bits, q [N][K/2] u8, s/b [N][K/G] fp16 bits -> y [R][N]."""
    x, q, s, b = _c(x, np.uint16), _c(q, np.uint8), _c(s, np.uint16), _c(b, np.uint16)
    R, K = x.shape
    N = q.shape[0]
    assert q.shape == (N, K // 2) and s.shape == (N, K // G) and b.shape == s.shape
    L = lib()
    if out_f32:
        y = np.empty((R, N), np.float32)
        L.ov_w4_linear_f32(ptr(x, np.uint16), R, K, ptr(q, np.uint8), ptr(s, np.uint16),
                           ptr(b, np.uint16), N, G, ptr(y, np.float32))
    else:
        y = np.empty((R, N), np.float64)
        L.ov_w4_linear(ptr(x, np.uint16), R, K, ptr(q, np.uint8), ptr(s, np.uint16),
                       ptr(b, np.uint16), N, G, ptr(y, np.float64))
    return y


def w4_linear_fp32(x, q, s, b, G):
    """The linear evaluated in fp32 arithmetic, two-level order (per group in
    ascending k, then the groups in ascending order) -> y [R][N] fp32."""
    x, q, s, b = _c(x, np.uint16), _c(q, np.uint8), _c(s, np.uint16), _c(b, np.uint16)
    R, K = x.shape
    N = q.shape[0]
    assert q.shape == (N, K // 2) and s.shape == (N, K // G) and b.shape == s.shape
    y = np.empty((R, N), np.float32)
    lib().ov_w4_linear_fp32(ptr(x, np.uint16), R, K, ptr(q, np.uint8), ptr(s, np.uint16),
                            ptr(b, np.uint16), N, G, ptr(y, np.float32))
    return y


def e2m1_to_f64(code):
    return float(lib().ov_e2m1_to_f64(int(code)))


def e4m3_to_f64(b):
    return float(lib().ov_e4m3_to_f64(int(b)))


def nvfp4_linear(x, q, s, s_t, out_f32=True):
    """x [R][K] bf16 bits, q [N][K/2] u8 (E2M1 pairs, low nibble = even k),
    s [N][K/16] u8 (E4M3 block scales), s_t fp32 tensor scale -> y [R][N] fp32."""
    x, q, s = _c(x, np.uint16), _c(q, np.uint8), _c(s, np.uint8)
    R, K = x.shape
    N = q.shape[0]
    assert q.shape == (N, K // 2) and s.shape == (N, K // 16)
    y = np.empty((R, N), np.float32)
    lib().ov_nvfp4_linear_f32(ptr(x, np.uint16), R, K, ptr(q, np.uint8), ptr(s, np.uint8), float(s_t), N,
                              ptr(y, np.float32))
    return y


def silu_mul_bf16(g, u):
    g, u = _c(g, np.float32), _c(u, np.float32)
    assert g.shape == u.shape
    h = np.empty(g.shape, np.uint16)
    lib().ov_silu_mul_bf16(ptr(g, np.float32), ptr(u, np.float32), g.size, ptr(h, np.uint16))
    return h


def mlp(x, gate, up, down, G):
    """gate/up/down are (q, s, b) triples.  Returns y, g, u, h."""
    x = _c(x, np.uint16)
    R, H = x.shape
    I = gate[0].shape[0]
    t = [_c(a, d) for w in (gate, up, down) for a, d in zip(w, (np.uint8, np.uint16, np.uint16))]
    assert t[0].shape == (I, H // 2) and t[6].shape == (H, I // 2)
    y = np.empty((R, H), np.float32)
    g = np.empty((R, I), np.float32)
    u = np.empty((R, I), np.float32)
    h = np.empty((R, I), np.uint16)
    lib().ov_mlp(ptr(x, np.uint16), R, H, I, G,
                 *[ptr(a, a.dtype) for a in t],
                 ptr(y, np.float32), ptr(g, np.float32), ptr(u, np.float32), ptr(h, np.uint16))
    return y, g, u, h


# --- sampler, accept -------------------------------------------------------

def topk(logits_row, k):
    l = _c(logits_row, np.float32)
    ids = np.empty(min(k, l.size), np.int32)
    n = lib().ov_topk(ptr(l, np.float32), l.size, k, ptr(ids, np.int32))
    return ids[:n]


def sample_from_candidates(logits_row, cand, pos, T, top_p, seed):
    l = _c(logits_row, np.float32)
    c = _c(cand, np.int32)
    o = SampleOut()
    lib().ov_sample_from_candidates(ptr(l, np.float32), ptr(c, np.int32), c.size, int(pos),
                                    float(T), float(top_p), C.c_uint64(seed), C.byref(o))
    return o


def sample_row(logits_row, pos, T, top_k, top_p, seed):
    l = _c(logits_row, np.float32)
    o = SampleOut()
    lib().ov_sample_row(ptr(l, np.float32), l.size, int(pos), float(T), int(top_k),
                        float(top_p), C.c_uint64(seed), C.byref(o))
    return o


def sample_rows(logits, positions, T, top_k, top_p, seed):
    """Returns tokens [R] i32, gaps [R] f64, n_kept [R], topp_edge [R]."""
    l = _c(logits, np.float32)
    R, V = l.shape
    p = _c(positions, np.int64)
    assert p.shape == (R,)
    tok = np.empty(R, np.int32)
    gap = np.empty(R, np.float64)
    kept = np.empty(R, np.int32)
    edge = np.empty(R, np.int32)
    lib().ov_sample_rows(ptr(l, np.float32), R, V, ptr(p, np.int64), float(T), int(top_k),
                         float(top_p), C.c_uint64(seed), ptr(tok, np.int32),
                         ptr(gap, np.float64), ptr(kept, np.int32), ptr(edge, np.int32))
    return tok, gap, kept, edge


def sample_many(logits_row, positions, seeds, T, top_k, top_p):
    l = _c(logits_row, np.float32)
    p = _c(positions, np.int64)
    sd = _c(seeds, np.uint64)
    assert p.shape == sd.shape
    tok = np.empty(p.size, np.int32)
    lib().ov_sample_many(ptr(l, np.float32), l.size, p.size, ptr(p, np.int64),
                         sd.ctypes.data_as(C.POINTER(C.c_uint64)), float(T), int(top_k),
                         float(top_p), ptr(tok, np.int32))
    return tok


def accept(sampled, draft):
    s = _c(sampled, np.int32)
    d = _c(draft, np.int32)
    a = C.c_int32()
    n = C.c_int32()
    lib().ov_accept(ptr(s, np.int32), s.size, ptr(d, np.int32) if d.size else None,
                    d.size, C.byref(a), C.byref(n))
    return a.value, n.value


# --- MoE ---------------------------------------------------------------------

def moe_route(rho_row, top):
    r = _c(rho_row, np.float32)
    ids = np.empty(top, np.int32)
    w = np.empty(top, np.float64)
    lib().ov_moe_route(ptr(r, np.float32), r.size, top, ptr(ids, np.int32), ptr(w, np.float64))
    return ids, w


def moe(x, rho, top, G, gate, up, down):
    """Stacked experts: gate/up q [E][I][H/2], s/b [E][I][H/G]; down q [E][H][I/2]."""
    x = _c(x, np.uint16)
    rho = _c(rho, np.float32)
    R, H = x.shape
    E = rho.shape[1]
    I = gate[0].shape[1]
    t = [_c(a, d) for w in (gate, up, down) for a, d in zip(w, (np.uint8, np.uint16, np.uint16))]
    assert t[0].shape == (E, I, H // 2) and t[6].shape == (E, H, I // 2)
    y = np.empty((R, H), np.float32)
    ids = np.empty((R, top), np.int32)
    w = np.empty((R, top), np.float64)
    lib().ov_moe(ptr(x, np.uint16), ptr(rho, np.float32), R, H, I, E, top, G,
                 *[ptr(a, a.dtype) for a in t], ptr(y, np.float32), ptr(ids, np.int32),
                 ptr(w, np.float64))
    return y, ids, w


# --- decoder (oracle/decoder.c) ---------------------------------------------

from .decoder import Decoder, attend, draft_chain, drafted_decode, rmsnorm_bf16, rope, serial_decode  # noqa: E402,F401
