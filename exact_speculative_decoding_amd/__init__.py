"""Python binding of libexactverify.so, the MI355X verify pass of exact drafted
decoding.  Argument marshalling only: every step runs in the HIP kernels of
the library; PyTorch supplies device memory and the current stream.

The functions mirror the C ABI in include/exactverify.h and take torch tensors
on the current HIP device.  bf16 / fp16 data may be passed as torch.bfloat16 /
torch.float16 tensors or as int16/uint16 bit patterns.

There is no fallback: if the library is not built, or no GPU is visible,
calls raise.
"""
import ctypes as C
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libexactverify.so")

EV_OK, EV_EINVAL, EV_EUNSUPPORTED, EV_EHIP, EV_EWORKSPACE = 0, -1, -2, -3, -4
MAX_LANES = 16
MAX_TOPK = 64

_lib = None


class EvError(RuntimeError):
    def __init__(self, code, msg):
        super().__init__(f"[{code}] {msg}")
        self.code = code


class Sampling(C.Structure):
    _fields_ = [("temperature", C.c_double), ("top_k", C.c_int32), ("top_p", C.c_double),
                ("seed", C.c_uint64)]


class DecoderConfig(C.Structure):
    _fields_ = [("layers", C.c_int32), ("hidden", C.c_int32), ("heads", C.c_int32),
                ("kv_heads", C.c_int32), ("head_dim", C.c_int32), ("intermediate", C.c_int32),
                ("vocab", C.c_int32), ("group", C.c_int32), ("rope_base", C.c_double),
                ("rms_eps", C.c_double)]


class DecoderLayer(C.Structure):
    _fields_ = [("attn_norm", C.c_void_p), ("w_qkv", C.c_void_p), ("w_o", C.c_void_p),
                ("mlp_norm", C.c_void_p), ("w_gate", C.c_void_p), ("w_up", C.c_void_p),
                ("w_down", C.c_void_p)]


class DecoderWeights(C.Structure):
    _fields_ = [("embed", C.c_void_p), ("layers", C.POINTER(DecoderLayer)),
                ("final_norm", C.c_void_p), ("w_lm", C.c_void_p)]


_vp, _sz, _i32, _i64 = C.c_void_p, C.c_size_t, C.c_int32, C.c_int64

# name -> (restype, argtypes)
_SIGS = {
    "ev_last_error": (C.c_char_p, []),
    "ev_version": (_i32, []),
    "w4_packed_bytes": (_sz, [_i32, _i32, _i32]),
    "w4_pack": (_i32, [_vp, _vp, _vp, _i32, _i32, _i32, _vp, _sz, _vp]),
    "verify_linear_w4_workspace": (_sz, [_i32, _i32, _i32]),
    "verify_linear_w4": (_i32, [_vp, _i32, _i32, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
    "verify_linear_w4_standard_workspace": (_sz, [_i32, _i32, _i32]),
    "verify_linear_w4_standard": (_i32, [_vp, _i32, _i32, _vp, _vp, _vp, _i32, _i32, _vp, _vp, _sz, _vp]),
    "nvfp4_packed_bytes": (_sz, [_i32, _i32]),
    "nvfp4_pack": (_i32, [_vp, _vp, _i32, _i32, _vp, _sz, _vp]),
    "verify_linear_nvfp4_workspace": (_sz, [_i32, _i32]),
    "verify_linear_nvfp4": (_i32, [_vp, _i32, _i32, _vp, _i32, C.c_float, _vp, _vp, _sz, _vp]),
    "verify_mlp_w4_workspace": (_sz, [_i32, _i32, _i32]),
    "verify_mlp_w4": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp, _sz,
                             _vp]),
    "verify_mlp_w4_noalloc": (_i32, [_vp, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp, _vp]),
    "verify_moe_w4_workspace": (_sz, [_i32, _i32, _i32, _i32, _i32]),
    "verify_moe_w4": (_i32, [_vp, _vp, _i32, _i32, _i32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _vp,
                             _vp, _vp, _sz, _vp]),
    "keyed_sample_workspace": (_sz, [_i32]),
    "keyed_sample": (_i32, [_vp, _i32, _i32, _vp, Sampling, _vp, _vp, _vp, _sz, _vp]),
    "accept_prefix": (_i32, [_vp, _i32, _vp, _i32, _vp, _vp, _vp]),
    "toy_decoder_create": (_i32, [C.POINTER(DecoderConfig), C.POINTER(DecoderWeights), _vp, _vp, _i32,
                                  C.POINTER(_vp)]),
    "toy_decoder_destroy": (None, [_vp]),
    "verify_step_workspace": (_sz, [_vp]),
    "verify_step": (_i32, [_vp, _vp, _i32, _i64, Sampling, _vp, _vp, _vp, _vp, _sz, _vp]),
    "verify_step_host": (_i32, [_vp, _vp, _i32, _i64, Sampling, _vp, _vp, _vp, _sz, _vp]),
    "ev_read_probe": (_i32, [_vp, _sz, _vp, _vp]),
    "toy_decoder_set_graphs": (_i32, [_vp, _i32]),
    "toy_decoder_graph_stats": (_i32, [_vp, C.POINTER(_i64), C.POINTER(_i32)]),
    "toy_decoder_prefill": (_i32, [_vp, _vp, _i32, _i64, _i32, _vp, _sz, _vp]),
    "toy_decoder_draft_workspace": (_sz, [_vp]),
    "toy_decoder_draft": (_i32, [_vp, _vp, _vp, _vp, _i32, C.c_double, _vp, _vp, _vp, _vp, _sz, _vp]),
    "verify_probe_workspace": (_sz, [_vp]),
    "verify_probe": (_i32, [_vp, _vp, _i32, _i64, Sampling, _vp, _vp, _sz, _vp]),
    "ev_w4_timing": (_i32, [_i32]),
    "ev_w4_timing_read": (_i32, [C.POINTER(_i64), C.POINTER(C.c_double), C.POINTER(C.c_double)]),
    "ev_w4_timing_stamps": (_i32, [_vp, _i64, _vp, _i32, C.POINTER(_i32)]),
}


def lib():
    """Load the library (raises if it has not been built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(LIB_PATH):
            raise RuntimeError(f"{LIB_PATH} is not built: run `python __graft_entry__.py` "
                               "(build()) or `python exact_speculative_decoding_amd/build.py`")
        L = C.CDLL(LIB_PATH)
        for name, (res, args) in _SIGS.items():
            f = getattr(L, name)
            f.restype = res
            f.argtypes = args
        _lib = L
    return _lib


def exported_symbols():
    return list(_SIGS)


def _check(rc):
    if rc != EV_OK:
        raise EvError(rc, lib().ev_last_error().decode(errors="replace"))


def _stream(stream):
    if stream is None:
        stream = torch.cuda.current_stream()
    return C.c_void_p(stream.cuda_stream if hasattr(stream, "cuda_stream") else int(stream))


def _dev(t, name, dtypes):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name}: expected a torch tensor")
    if not t.is_cuda:
        raise ValueError(f"{name}: must be a device tensor")
    if t.dtype not in dtypes:
        raise TypeError(f"{name}: dtype {t.dtype} not in {dtypes}")
    if not t.is_contiguous():
        raise ValueError(f"{name}: must be contiguous")
    return C.c_void_p(t.data_ptr())


_B16 = (torch.bfloat16, torch.int16, torch.uint16)
_F16 = (torch.float16, torch.int16, torch.uint16)
_U8 = (torch.uint8,)


def _workspace(nbytes, device, ws):
    if nbytes == 0:
        return None, 0
    if ws is None:
        ws = torch.empty(nbytes, dtype=torch.uint8, device=device)
    if ws.numel() * ws.element_size() < nbytes:
        raise ValueError(f"workspace too small: {ws.numel()} < {nbytes}")
    return ws, ws.numel() * ws.element_size()


class PackedW4:
    """A W4 matrix in the packed layout (device bytes) with its shape."""

    def __init__(self, blob, N, K, G):
        self.blob, self.N, self.K, self.G = blob, N, K, G


def w4_packed_bytes(N, K, G):
    return int(lib().w4_packed_bytes(N, K, G))


def w4_pack(q, s, b, G, out=None, stream=None):
    """Pack a standard-layout matrix q [N][K/2] u8, s/b [N][K/G] fp16 (device)."""
    N, Kh = q.shape
    K = 2 * Kh
    nb = w4_packed_bytes(N, K, G)
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=q.device)
    _check(lib().w4_pack(_dev(q, "q", _U8), _dev(s, "s", _F16), _dev(b, "b", _F16), N, K, G,
                         _dev(out, "packed", _U8), out.numel(), _stream(stream)))
    return PackedW4(out, N, K, G)


def verify_linear_w4_workspace(K, N, G):
    return int(lib().verify_linear_w4_workspace(K, N, G))


def verify_linear_w4(x, w, y=None, ws=None, stream=None):
    """y[R][N] fp32 = W4 linear of x[R][K] (bf16) with the packed matrix w."""
    R, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, the matrix K={w.K}")
    if y is None:
        y = torch.empty((R, w.N), dtype=torch.float32, device=x.device)
    ws, nb = _workspace(verify_linear_w4_workspace(K, w.N, w.G), x.device, ws)
    _check(lib().verify_linear_w4(
        _dev(x, "x", _B16), R, K, _dev(w.blob, "w", _U8), w.N, w.G,
        _dev(y, "y", (torch.float32,)),
        None if ws is None else C.c_void_p(ws.data_ptr()), nb, _stream(stream)))
    return y


def verify_linear_w4_standard_workspace(K, N, G):
    return int(lib().verify_linear_w4_standard_workspace(K, N, G))


def verify_linear_w4_standard(x, q, s, b, G, y=None, ws=None, stream=None):
    """y[R][N] fp32 = W4 linear of x[R][K] (bf16) with the standard-layout
    matrix q [N][K/2] u8, s/b [N][K/G] fp16 (packed inside the call)."""
    R, K = x.shape
    N, Kh = q.shape
    if 2 * Kh != K:
        raise ValueError(f"x has K={K}, the matrix K={2 * Kh}")
    if y is None:
        y = torch.empty((R, N), dtype=torch.float32, device=x.device)
    ws, nb = _workspace(verify_linear_w4_standard_workspace(K, N, G), x.device, ws)
    _check(lib().verify_linear_w4_standard(
        _dev(x, "x", _B16), R, K, _dev(q, "q", _U8), _dev(s, "s", _F16), _dev(b, "b", _F16), N, G,
        _dev(y, "y", (torch.float32,)), None if ws is None else C.c_void_p(ws.data_ptr()), nb, _stream(stream)))
    return y


class PackedNvfp4:
    """An NVFP4-style matrix in the packed layout (device bytes), its shape and
    tensor scale."""

    def __init__(self, blob, N, K, tensor_scale):
        self.blob, self.N, self.K, self.tensor_scale = blob, N, K, float(tensor_scale)


def nvfp4_pack(q, s, tensor_scale, out=None, stream=None):
    """Pack q [N][K/2] u8 (E2M1 pairs) and s [N][K/16] u8 (E4M3), device."""
    N, Kh = q.shape
    K = 2 * Kh
    nb = int(lib().nvfp4_packed_bytes(N, K))
    if out is None:
        out = torch.empty(nb, dtype=torch.uint8, device=q.device)
    _check(lib().nvfp4_pack(_dev(q, "q", _U8), _dev(s, "s", _U8), N, K, _dev(out, "packed", _U8), out.numel(),
                            _stream(stream)))
    return PackedNvfp4(out, N, K, tensor_scale)


def verify_linear_nvfp4(x, w, y=None, ws=None, stream=None):
    """y[R][N] fp32 = the NVFP4 linear of x[R][K] (bf16) with the packed matrix w."""
    R, K = x.shape
    if K != w.K:
        raise ValueError(f"x has K={K}, the matrix K={w.K}")
    if y is None:
        y = torch.empty((R, w.N), dtype=torch.float32, device=x.device)
    ws, nb = _workspace(int(lib().verify_linear_nvfp4_workspace(K, w.N)), x.device, ws)
    _check(lib().verify_linear_nvfp4(
        _dev(x, "x", _B16), R, K, _dev(w.blob, "w", _U8), w.N, C.c_float(w.tensor_scale),
        _dev(y, "y", (torch.float32,)), None if ws is None else C.c_void_p(ws.data_ptr()), nb, _stream(stream)))
    return y


def verify_mlp_w4_workspace(H, I, G):
    return int(lib().verify_mlp_w4_workspace(H, I, G))


def verify_mlp_w4(x, gate, up, down, y=None, h=None, ws=None, stream=None):
    """Dense SiLU-gated MLP slice on packed gate/up (I x H) and down (H x I)."""
    R, H = x.shape
    I, G = gate.N, gate.G
    if not (gate.K == up.K == down.N == H and up.N == down.K == I and up.G == down.G == G):
        raise ValueError("inconsistent MLP matrix shapes")
    if y is None:
        y = torch.empty((R, H), dtype=torch.float32, device=x.device)
    ws, nb = _workspace(verify_mlp_w4_workspace(H, I, G), x.device, ws)
    _check(lib().verify_mlp_w4(
        _dev(x, "x", _B16), R, H, I, G, _dev(gate.blob, "gate", _U8), _dev(up.blob, "up", _U8),
        _dev(down.blob, "down", _U8), _dev(y, "y", (torch.float32,)),
        None if h is None else _dev(h, "h", _B16),
        C.c_void_p(ws.data_ptr()), nb, _stream(stream)))
    return y


def verify_mlp_w4_noalloc(x, gate, up, down, y, h=None, stream=None):
    """verify_mlp_w4 on the library's own device scratch (no workspace; the
    caller passes the output y [R][H] fp32, and optionally h [R][I] bf16)."""
    R, H = x.shape
    I, G = gate.N, gate.G
    if not (gate.K == up.K == down.N == H and up.N == down.K == I and up.G == down.G == G):
        raise ValueError("inconsistent MLP matrix shapes")
    _check(lib().verify_mlp_w4_noalloc(
        _dev(x, "x", _B16), R, H, I, G, _dev(gate.blob, "gate", _U8), _dev(up.blob, "up", _U8),
        _dev(down.blob, "down", _U8), _dev(y, "y", (torch.float32,)),
        None if h is None else _dev(h, "h", _B16), _stream(stream)))
    return y


class PackedW4Stack:
    """E W4 matrices of one shape, packed back to back (expert e at e * nbytes)."""

    def __init__(self, blob, E, N, K, G):
        self.blob, self.E, self.N, self.K, self.G = blob, E, N, K, G
        self.nbytes = w4_packed_bytes(N, K, G)


def w4_pack_stack(q, s, b, G, stream=None):
    """Pack E standard-layout matrices q [E][N][K/2] u8, s/b [E][N][K/G] fp16."""
    E, N, Kh = q.shape
    K = 2 * Kh
    nb = w4_packed_bytes(N, K, G)
    out = torch.empty(E * nb, dtype=torch.uint8, device=q.device)
    for e in range(E):
        w4_pack(q[e], s[e], b[e], G, out=out[e * nb:(e + 1) * nb], stream=stream)
    return PackedW4Stack(out, E, N, K, G)


def verify_moe_w4_workspace(H, I, E, top, G):
    return int(lib().verify_moe_w4_workspace(H, I, E, top, G))


def verify_moe_w4(x, router, gate, up, down, top, y=None, expert_ids=None, expert_w=None, ws=None,
                  stream=None):
    """MoE verify layer: x [R][H] bf16, router [R][E] fp32, stacks of packed
    experts (gate/up I x H, down H x I).  Returns y [R][H] fp32."""
    R, H = x.shape
    E, I, G = gate.E, gate.N, gate.G
    if not (gate.K == up.K == down.N == H and up.N == down.K == I and up.E == down.E == E
            and up.G == down.G == G and router.shape == (R, E)):
        raise ValueError("inconsistent MoE shapes")
    if y is None:
        y = torch.empty((R, H), dtype=torch.float32, device=x.device)
    ws, nb = _workspace(verify_moe_w4_workspace(H, I, E, top, G), x.device, ws)
    _check(lib().verify_moe_w4(
        _dev(x, "x", _B16), _dev(router, "router", (torch.float32,)), R, H, I, E, top, G,
        _dev(gate.blob, "gate", _U8), _dev(up.blob, "up", _U8), _dev(down.blob, "down", _U8),
        _dev(y, "y", (torch.float32,)),
        None if expert_ids is None else _dev(expert_ids, "expert_ids", (torch.int32,)),
        None if expert_w is None else _dev(expert_w, "expert_w", (torch.float32,)),
        None if ws is None else C.c_void_p(ws.data_ptr()), nb, _stream(stream)))
    return y


def keyed_sample_workspace(V):
    return int(lib().keyed_sample_workspace(V))


def keyed_sample(logits, positions, temperature, top_k, top_p, seed, tokens=None, gap=None,
                 ws=None, stream=None):
    """tokens [R] int32 (and gap [R] fp64 if given) for logits [R][V] fp32."""
    R, V = logits.shape
    if tokens is None:
        tokens = torch.empty(R, dtype=torch.int32, device=logits.device)
    ws, nb = _workspace(keyed_sample_workspace(V), logits.device, ws)
    sp = Sampling(float(temperature), int(top_k), float(top_p), int(seed) & ((1 << 64) - 1))
    _check(lib().keyed_sample(
        _dev(logits, "logits", (torch.float32,)), R, V, _dev(positions, "positions", (torch.int64,)),
        sp, _dev(tokens, "tokens", (torch.int32,)),
        None if gap is None else _dev(gap, "gap", (torch.float64,)),
        C.c_void_p(ws.data_ptr()), nb, _stream(stream)))
    return tokens


def accept_prefix(sampled, draft, n_accept=None, n_commit=None, stream=None):
    """(n_accept, n_commit) as one-element int32 device tensors."""
    R = sampled.shape[0]
    D = 0 if draft is None else draft.shape[0]
    dev = sampled.device
    if n_accept is None:
        n_accept = torch.empty(1, dtype=torch.int32, device=dev)
    if n_commit is None:
        n_commit = torch.empty(1, dtype=torch.int32, device=dev)
    _check(lib().accept_prefix(
        _dev(sampled, "sampled", (torch.int32,)), R,
        None if D == 0 else _dev(draft, "draft", (torch.int32,)), D,
        _dev(n_accept, "n_accept", (torch.int32,)), _dev(n_commit, "n_commit", (torch.int32,)),
        _stream(stream)))
    return n_accept, n_commit


class ToyDecoder:
    """A decoder whose weights and K/V caches live on the device, driven by
    verify_step.  `weights` holds device tensors: embed [V][H] bf16,
    final_norm [H] fp32, lm (PackedW4), and per layer (list `layers` of dicts)
    attn_norm, mlp_norm [H] fp32 and packed qkv, o, gate, up, down.  The caches
    are [layers][kv_heads][max_ctx][128] fp16 device tensors, the value cache
    in the blocked slot order (v_cache_blocked)."""

    def __init__(self, cfg, weights, k_cache, v_cache):
        self.cfg = cfg
        self.weights, self.k_cache, self.v_cache = weights, k_cache, v_cache
        self.max_ctx = int(k_cache.shape[2])
        c = DecoderConfig(cfg["layers"], cfg["hidden"], cfg["heads"], cfg["kv_heads"],
                          cfg["head_dim"], cfg["inter"], cfg["vocab"], cfg["G"],
                          float(cfg["rope_base"]), float(cfg["eps"]))
        L = weights["layers"]
        self._layers = (DecoderLayer * len(L))(*[
            DecoderLayer(_dev(y["attn_norm"], "attn_norm", (torch.float32,)).value,
                         _dev(y["qkv"].blob, "qkv", _U8).value, _dev(y["o"].blob, "o", _U8).value,
                         _dev(y["mlp_norm"], "mlp_norm", (torch.float32,)).value,
                         _dev(y["gate"].blob, "gate", _U8).value, _dev(y["up"].blob, "up", _U8).value,
                         _dev(y["down"].blob, "down", _U8).value) for y in L])
        w = DecoderWeights(_dev(weights["embed"], "embed", _B16).value, self._layers,
                           _dev(weights["final_norm"], "final_norm", (torch.float32,)).value,
                           _dev(weights["lm"].blob, "lm", _U8).value)
        h = C.c_void_p()
        _check(lib().toy_decoder_create(C.byref(c), C.byref(w), _dev(k_cache, "k_cache", _F16),
                                        _dev(v_cache, "v_cache", _F16), self.max_ctx, C.byref(h)))
        self._h = h
        self._outs = {}  # R -> (sampled, n_commit) kept for graph replay
        self._host_io = {}  # R -> buffers of verify_step_host
        self.ws = torch.empty(int(lib().verify_step_workspace(h)), dtype=torch.uint8,
                              device=k_cache.device)

    def v_cache_standard(self):
        """The value cache in the plain [layers][kv_heads][C][128] order."""
        return v_cache_standard(self.v_cache)

    def __del__(self):
        h = getattr(self, "_h", None)
        if h is not None and h.value and _lib is not None:
            _lib.toy_decoder_destroy(h)
            self._h = None

    def set_graphs(self, enable):
        """Graph replay of verify_step on or off (on by default)."""
        _check(lib().toy_decoder_set_graphs(self._h, 1 if enable else 0))

    def draft(self, head, n_commit, sampled, max_drafts, min_conf, drafts, n_drafts, stream=None):
        """The MTP-style draft chain after a verify step (device tensors: the
        step's n_commit [1] and sampled [R]; outputs drafts [max_drafts] and
        n_drafts [1] int32)."""
        if getattr(self, "_dws", None) is None:
            self._dws = torch.empty(int(lib().toy_decoder_draft_workspace(self._h)), dtype=torch.uint8,
                                    device=self.ws.device)
        _check(lib().toy_decoder_draft(
            self._h, _dev(head.blob, "w_draft", _U8), _dev(n_commit, "n_commit", (torch.int32,)),
            _dev(sampled, "sampled", (torch.int32,)), int(max_drafts), float(min_conf),
            _dev(drafts, "drafts", (torch.int32,)), _dev(n_drafts, "n_drafts", (torch.int32,)),
            C.c_void_p(self.ws.data_ptr()), C.c_void_p(self._dws.data_ptr()), self._dws.numel(),
            _stream(stream)))

    def verify_and_draft_host(self, tokens, pos0, temperature, top_k, top_p, seed, head, max_drafts,
                              min_conf=0.3):
        """One round for a host loop with an MTP-style head: verify `tokens`
        (a list), then draft the next round's tokens from the last committed
        row.  One upload, one read-back; returns (sampled tokens, n_commit,
        the next round's drafts)."""
        R = len(tokens)
        key = ("mtp", R, max_drafts)
        io = self._host_io.get(key)
        if io is None:
            dev = self.ws.device
            n = R + 2 + max_drafts
            io = (torch.empty(R, dtype=torch.int32, pin_memory=True), torch.empty(R, dtype=torch.int32, device=dev),
                  torch.empty(n, dtype=torch.int32, device=dev), torch.empty(n, dtype=torch.int32, pin_memory=True))
            self._host_io[key] = io
        tok_h, tok_d, out_d, out_h = io
        tok_h.numpy()[:] = tokens
        tok_d.copy_(tok_h, non_blocking=True)
        sampled, n_commit = out_d[:R], out_d[R:R + 1]
        drafts, n_drafts = out_d[R + 1:R + 1 + max_drafts], out_d[R + 1 + max_drafts:]
        self.verify_step(tok_d, pos0, temperature, top_k, top_p, seed, sampled=sampled, n_commit=n_commit)
        self.draft(head, n_commit, sampled, max_drafts, min_conf, drafts, n_drafts)
        out_h.copy_(out_d, non_blocking=True)
        torch.cuda.current_stream(self.ws.device).synchronize()
        o = out_h.numpy()
        nd = int(o[R + 1 + max_drafts])
        return o[:R].tolist(), int(o[R]), o[R + 1:R + 1 + nd].tolist()

    def prefill(self, tokens, pos0, grid=2048, stream=None):
        """Write the cache entries of slots pos0.. for tokens [n] int32 (device),
        in grid-aligned passes of at most 16 rows."""
        n = tokens.shape[0]
        _check(lib().toy_decoder_prefill(self._h, _dev(tokens, "tokens", (torch.int32,)) if n else None, n,
                                         int(pos0), int(grid), C.c_void_p(self.ws.data_ptr()), self.ws.numel(),
                                         _stream(stream)))

    def verify_probe(self, tokens, pos0, temperature, top_k, top_p, seed, stream=None):
        """Words that differ between an R-row verify step over tokens [R] int32
        (device) at slots pos0.. and the same rows stepped one at a time
        (logits, sampled tokens, cache entries); 0 when R-row passes are exact.
        Writes the cache slots pos0..pos0+R-1."""
        R = tokens.shape[0]
        ws = torch.empty(int(lib().verify_probe_workspace(self._h)), dtype=torch.uint8, device=tokens.device)
        out = torch.empty(1, dtype=torch.int32, device=tokens.device)
        sp = Sampling(float(temperature), int(top_k), float(top_p), int(seed) & ((1 << 64) - 1))
        _check(lib().verify_probe(self._h, _dev(tokens, "tokens", (torch.int32,)), R, int(pos0), sp,
                                  _dev(out, "mismatch", (torch.int32,)), C.c_void_p(ws.data_ptr()),
                                  ws.numel(), _stream(stream)))
        return int(out.cpu()[0])

    def graph_stats(self):
        """(steps captured since creation, captured steps held now)."""
        n, k = C.c_int64(), C.c_int32()
        _check(lib().toy_decoder_graph_stats(self._h, C.byref(n), C.byref(k)))
        return n.value, k.value

    def verify_step(self, tokens, pos0, temperature, top_k, top_p, seed, sampled=None,
                    n_commit=None, logits=None, stream=None):
        """One verify pass over tokens [R] int32 (device) at slots pos0..; returns
        (sampled [R] int32, n_commit [1] int32), device tensors.  Without
        caller buffers the results land in buffers this handle keeps per R, so
        that the captured step is replayed; the next call with the same R
        overwrites them."""
        R = tokens.shape[0]
        dev = tokens.device
        if sampled is None or n_commit is None:
            outs = self._outs.get(R)
            if outs is None:
                outs = (torch.empty(R, dtype=torch.int32, device=dev), torch.empty(1, dtype=torch.int32, device=dev))
                self._outs[R] = outs
            sampled = outs[0] if sampled is None else sampled
            n_commit = outs[1] if n_commit is None else n_commit
        sp = Sampling(float(temperature), int(top_k), float(top_p), int(seed) & ((1 << 64) - 1))
        _check(lib().verify_step(
            self._h, _dev(tokens, "tokens", (torch.int32,)), R, int(pos0), sp,
            _dev(sampled, "sampled", (torch.int32,)), _dev(n_commit, "n_commit", (torch.int32,)),
            None if logits is None else _dev(logits, "logits", (torch.float32,)),
            C.c_void_p(self.ws.data_ptr()), self.ws.numel(), _stream(stream)))
        return sampled, n_commit


    def verify_step_host(self, tokens, pos0, temperature, top_k, top_p, seed, stream=None):
        """verify_step for a host round loop: `tokens` is a list of R ints;
        returns (sampled tokens as a list, n_commit).  One native call: the
        tokens go to the step's first kernel as an argument, the results come
        back in one copy, and the call waits for the stream."""
        R = len(tokens)
        io = self._host_io.get(("native", R))
        if io is None:
            io = ((C.c_int32 * R)(), (C.c_int32 * R)(), C.c_int32())
            self._host_io[("native", R)] = io
        tok, smp, nc = io
        tok[:] = [int(t) for t in tokens]
        sp = Sampling(float(temperature), int(top_k), float(top_p), int(seed) & ((1 << 64) - 1))
        _check(lib().verify_step_host(self._h, tok, R, int(pos0), sp, smp, C.byref(nc),
                                      C.c_void_p(self.ws.data_ptr()), self.ws.numel(), _stream(stream)))
        return list(smp), int(nc.value)


# Value-cache slot order inside a block of 32 slots (see verify_step in
# include/exactverify.h): slot s sits at position VSLOT_POS[s].
VSLOT_POS = [8 * (s // 4) + s % 4 if s < 16 else 8 * ((s - 16) // 4) + 4 + s % 4 for s in range(32)]
_VSLOT_AT = [VSLOT_POS.index(k) for k in range(32)]


def v_cache_blocked(v):
    """[layers][kv_heads][C][128] -> the blocked layout [layers][kv_heads][C/32][128][32]
    (numpy array or torch tensor)."""
    L, KV, C, D = v.shape
    x = v.reshape(L, KV, C // 32, 32, D)[:, :, :, _VSLOT_AT, :]
    return x.swapaxes(-1, -2).reshape(L, KV, C, D)


def v_cache_standard(vb):
    """Inverse of v_cache_blocked."""
    L, KV, C, D = vb.shape
    x = vb.reshape(L, KV, C // 32, D, 32).swapaxes(-1, -2)
    return x[:, :, :, VSLOT_POS, :].reshape(L, KV, C, D)


def load_decoder(cfg, w, kc, vc, device="cuda"):
    """Upload a decoder given in standard layouts (numpy: embed [V][H] bf16 bits,
    norms fp32, W4 q/s/b per matrix stacked over layers, caches fp16 bits) and
    pack its matrices; returns a ToyDecoder."""
    import numpy as np

    def t(a):
        a = np.ascontiguousarray(a)
        if a.dtype == np.uint16:
            a = a.view(np.int16)
        return torch.from_numpy(a).to(device)

    def pack(name, l=None):
        q, s_, b = (w[name + p] if l is None else w[name + p][l] for p in ("_q", "_s", "_b"))
        return w4_pack(t(q), t(s_), t(b), cfg["G"])

    layers = [dict(attn_norm=t(w["attn_norm"][l]), mlp_norm=t(w["mlp_norm"][l]),
                   qkv=pack("qkv", l), o=pack("o", l), gate=pack("gate", l), up=pack("up", l),
                   down=pack("down", l)) for l in range(cfg["layers"])]
    weights = dict(embed=t(w["embed"]), final_norm=t(w["final_norm"]), lm=pack("lm"), layers=layers)
    return ToyDecoder(cfg, weights, t(kc), t(np.ascontiguousarray(v_cache_blocked(vc))))


def w4_timing(enable):
    """Turn the per-launch event timing of the W4 kernel on or off."""
    _check(lib().ev_w4_timing(1 if enable else 0))


def read_probe(buf, sink, stream=None):
    """One plain streaming read of the uint8 device tensor buf (the practical
    read ceiling; timed by the W4 timing hook when it is on)."""
    _check(lib().ev_read_probe(_dev(buf, "buf", _U8), buf.numel(), _dev(sink, "sink", (torch.int32,)),
                               _stream(stream)))


def w4_timing_read():
    """(launches, total_ms, total_algorithmic_bytes) since the last read."""
    n, ms, by = C.c_int64(), C.c_double(), C.c_double()
    _check(lib().ev_w4_timing_read(C.byref(n), C.byref(ms), C.byref(by)))
    return n.value, ms.value, by.value


def w4_timing_stamps(max_pairs=1 << 20, max_launches=1 << 14):
    """(per-launch workgroup counts, [workgroups][2] device wall-clock stamps)
    of the launches recorded since the last w4_timing_read (not reset)."""
    import numpy as np
    st = np.empty((max_pairs, 2), np.uint64)
    cnt = np.empty(max_launches, np.int32)
    n = C.c_int32()
    _check(lib().ev_w4_timing_stamps(st.ctypes.data, max_pairs, cnt.ctypes.data, max_launches, C.byref(n)))
    c = cnt[:n.value].copy()
    return c, st[:int(c.sum())].copy()

