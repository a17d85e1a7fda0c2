"""C-ABI contract checks that need no GPU: the library loads, exports every
function include/exactverify.h declares, and rejects bad arguments with the
documented codes before anything is launched (so these run anywhere)."""
import ctypes as C
import os
import re

import pytest

import exact_speculative_decoding_amd as ev

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
P = C.c_void_p(0x10000)  # never dereferenced: every call below fails validation


def _declared():
    names = set()
    for h in os.listdir(os.path.join(ROOT, "include")):
        if not h.endswith(".h"):
            continue
        src = open(os.path.join(ROOT, "include", h)).read()
        src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
        for m in re.finditer(r"^\s*(?:const\s+)?[A-Za-z_][A-Za-z0-9_]*\s*\*?\s*([a-z_][a-z0-9_]*)\s*\(",
                             src, flags=re.M):
            names.add(m.group(1))
    return names


def test_every_declared_function_is_exported():
    L = ev.lib()
    declared = _declared()
    assert {"verify_linear_w4", "keyed_sample", "accept_prefix"} <= declared
    for name in declared:
        assert hasattr(L, name), name
    assert set(ev.exported_symbols()) >= declared


def test_workspace_sizes_do_not_depend_on_rows():
    # the workspace functions take no R at all; check they are stable and sane
    assert ev.verify_linear_w4_workspace(256, 512, 64) >= 0
    assert ev.verify_linear_w4_workspace(17408, 5120, 64) > 16 * 5120 * 4
    assert ev.keyed_sample_workspace(151936) >= 16 * 38 * 64 * 8 + 16 * 6 * 2048 * 8
    assert ev.verify_mlp_w4_workspace(5120, 17408, 64) > 0


def _lin(**kw):
    a = dict(x=P, R=4, K=256, w=P, N=512, G=64, y=P, ws=P, nb=1 << 30)
    a.update(kw)
    L = ev.lib()
    return L.verify_linear_w4(a["x"], a["R"], a["K"], a["w"], a["N"], a["G"], a["y"], a["ws"],
                              a["nb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), ev.EV_EINVAL), (dict(R=17), ev.EV_EINVAL), (dict(K=0), ev.EV_EINVAL),
    (dict(N=0), ev.EV_EINVAL), (dict(K=100), ev.EV_EINVAL), (dict(K=96, G=64), ev.EV_EINVAL),
    (dict(G=128), ev.EV_EUNSUPPORTED), (dict(G=16), ev.EV_EUNSUPPORTED),
    (dict(x=None), ev.EV_EINVAL), (dict(w=None), ev.EV_EINVAL), (dict(y=None), ev.EV_EINVAL),
    (dict(x=C.c_void_p(0x10002)), ev.EV_EINVAL), (dict(w=C.c_void_p(0x10008)), ev.EV_EINVAL),
    (dict(K=17408, N=5120, ws=None), ev.EV_EWORKSPACE), (dict(K=17408, N=5120, nb=64), ev.EV_EWORKSPACE),
    (dict(K=17408, N=5120, ws=C.c_void_p(0x10010)), ev.EV_EINVAL),
    (dict(K=1 << 20, N=1 << 14), ev.EV_EUNSUPPORTED),
])
def test_linear_rejects_bad_arguments(kw, code):
    if "ws" in kw or "nb" in kw:  # these cases must need a workspace, or the call would launch
        assert ev.verify_linear_w4_workspace(kw["K"], kw["N"], 64) > 64
    assert _lin(**kw) == code
    assert ev.lib().ev_last_error()


def _lin_std(**kw):
    a = dict(x=P, R=4, K=256, q=P, s=P, b=P, N=512, G=64, y=P, ws=P, nb=1 << 30)
    a.update(kw)
    return ev.lib().verify_linear_w4_standard(a["x"], a["R"], a["K"], a["q"], a["s"], a["b"], a["N"], a["G"],
                                              a["y"], a["ws"], a["nb"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), ev.EV_EINVAL), (dict(R=17), ev.EV_EINVAL), (dict(K=100), ev.EV_EINVAL),
    (dict(G=16), ev.EV_EUNSUPPORTED), (dict(q=None), ev.EV_EINVAL), (dict(s=None), ev.EV_EINVAL),
    (dict(b=None), ev.EV_EINVAL), (dict(y=None), ev.EV_EINVAL), (dict(x=C.c_void_p(0x10002)), ev.EV_EINVAL),
    (dict(q=C.c_void_p(0x10002)), ev.EV_EINVAL), (dict(s=C.c_void_p(0x10001)), ev.EV_EINVAL),
    (dict(ws=None), ev.EV_EWORKSPACE), (dict(nb=1024), ev.EV_EWORKSPACE),
    (dict(ws=C.c_void_p(0x10010)), ev.EV_EINVAL),
])
def test_standard_layout_linear_rejects_bad_arguments(kw, code):
    """Every check of the pack and of the linear comes before either launches
    (the workspace always holds the packed matrix, so it is never empty)."""
    assert ev.verify_linear_w4_standard_workspace(256, 512, 64) >= ev.w4_packed_bytes(512, 256, 64)
    assert _lin_std(**kw) == code
    assert ev.lib().ev_last_error()


@pytest.mark.parametrize("args,code", [
    ((P, P, P, 0, 256, 64), ev.EV_EINVAL), ((P, P, P, 512, 100, 64), ev.EV_EINVAL),
    ((P, P, P, 512, 256, 48), ev.EV_EUNSUPPORTED), ((None, P, P, 512, 256, 64), ev.EV_EINVAL),
    ((C.c_void_p(0x10001), P, P, 512, 256, 64), ev.EV_EINVAL),
])
def test_pack_rejects_bad_arguments(args, code):
    q, s, b, N, K, G = args
    assert ev.lib().w4_pack(q, s, b, N, K, G, P, 1 << 30, None) == code
    assert ev.lib().w4_pack(P, P, P, 512, 256, 64, P, 16, None) == ev.EV_EINVAL


def test_packed_size_is_the_standard_size_when_aligned():
    for N, K, G in ((17408, 5120, 64), (5120, 17408, 64), (768, 2048, 32), (151936, 5120, 64)):
        assert ev.w4_packed_bytes(N, K, G) == N * K // 2 + 4 * N * (K // G)
    assert ev.w4_packed_bytes(17, 96, 32) == 2 * 1 * (1024 + 256)


def _samp(R=2, V=512, T=0.7, k=20, p=0.95, ws=P, nb=1 << 30, logits=P, pos=P, tok=P):
    sp = ev.Sampling(T, k, p, 42)
    return ev.lib().keyed_sample(logits, R, V, pos, sp, tok, None, ws, nb, None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), ev.EV_EINVAL), (dict(R=17), ev.EV_EINVAL), (dict(V=0), ev.EV_EINVAL),
    (dict(V=262145), ev.EV_EUNSUPPORTED), (dict(T=-1.0), ev.EV_EINVAL),
    (dict(T=float("inf")), ev.EV_EINVAL), (dict(T=float("nan")), ev.EV_EINVAL),
    (dict(k=-1), ev.EV_EINVAL), (dict(k=65), ev.EV_EUNSUPPORTED), (dict(p=0.0), ev.EV_EINVAL),
    (dict(p=1.5), ev.EV_EINVAL), (dict(ws=None), ev.EV_EWORKSPACE), (dict(nb=8), ev.EV_EWORKSPACE),
    (dict(logits=None), ev.EV_EINVAL), (dict(tok=None), ev.EV_EINVAL),
])
def test_sampler_rejects_bad_arguments(kw, code):
    assert _samp(**kw) == code


@pytest.mark.parametrize("R,D,draft,code", [(0, 0, P, ev.EV_EINVAL), (17, 0, P, ev.EV_EINVAL),
                                            (4, 5, P, ev.EV_EINVAL), (4, -1, P, ev.EV_EINVAL),
                                            (4, 2, None, ev.EV_EINVAL)])
def test_accept_rejects_bad_arguments(R, D, draft, code):
    assert ev.lib().accept_prefix(P, R, draft, D, P, P, None) == code


def test_binding_refuses_host_tensors():
    import torch
    x = torch.zeros(2, 256, dtype=torch.bfloat16)
    w = ev.PackedW4(torch.zeros(ev.w4_packed_bytes(512, 256, 64), dtype=torch.uint8), 512, 256, 64)
    with pytest.raises((ValueError, RuntimeError)):
        ev.verify_linear_w4(x, w, y=torch.zeros(2, 512))


def _moe(**kw):
    a = dict(x=P, rho=P, R=4, H=256, I=128, E=16, top=4, G=32, wg=P, wu=P, wd=P, y=P, ids=None,
             w=None, ws=None, nb=0)
    a.update(kw)
    return ev.lib().verify_moe_w4(a["x"], a["rho"], a["R"], a["H"], a["I"], a["E"], a["top"], a["G"],
                                  a["wg"], a["wu"], a["wd"], a["y"], a["ids"], a["w"], a["ws"], a["nb"],
                                  None)


@pytest.mark.parametrize("kw,code", [
    (dict(R=0), ev.EV_EINVAL), (dict(R=17), ev.EV_EINVAL), (dict(E=0), ev.EV_EUNSUPPORTED),
    (dict(E=257), ev.EV_EUNSUPPORTED), (dict(top=0), ev.EV_EUNSUPPORTED), (dict(top=9), ev.EV_EUNSUPPORTED),
    (dict(E=3, top=4), ev.EV_EUNSUPPORTED), (dict(G=16), ev.EV_EUNSUPPORTED), (dict(H=100), ev.EV_EINVAL),
    (dict(I=48, G=32), ev.EV_EINVAL), (dict(x=None), ev.EV_EINVAL), (dict(rho=None), ev.EV_EINVAL),
    (dict(wd=None), ev.EV_EINVAL), (dict(y=None), ev.EV_EINVAL), (dict(y=C.c_void_p(0x10004)), ev.EV_EINVAL),
    (dict(ids=C.c_void_p(0x10002)), ev.EV_EINVAL), (dict(), ev.EV_EWORKSPACE),
    (dict(nb=64, ws=P), ev.EV_EWORKSPACE),
])
def test_moe_rejects_bad_arguments(kw, code):
    assert _moe(**kw) == code
    assert ev.lib().ev_last_error()


def test_moe_workspace_depends_on_shapes_only():
    a = ev.verify_moe_w4_workspace(2048, 768, 128, 8, 32)
    assert a > 0 and a == ev.verify_moe_w4_workspace(2048, 768, 128, 8, 32)
    assert ev.verify_moe_w4_workspace(2048, 768, 128, 9, 32) == 0
    assert ev.verify_moe_w4_workspace(256, 128, 16, 4, 32) < a


def test_decoder_steps_reject_a_null_handle():
    sp = ev.Sampling(0.7, 20, 0.95, 1)
    toks, smp, nc = (C.c_int32 * 2)(1, 2), (C.c_int32 * 2)(), C.c_int32()
    assert ev.lib().verify_step_host(None, toks, 2, 0, sp, smp, C.byref(nc), P, 1, None) == ev.EV_EINVAL
    assert ev.lib().verify_step(None, P, 2, 0, sp, P, P, None, P, 1, None) == ev.EV_EINVAL
