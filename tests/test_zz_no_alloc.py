"""verify_mlp_w4_noalloc (the MLP slice on the library's own device scratch,
for callers that cannot allocate) against verify_mlp_w4 with a caller
workspace: y and h bit-identical, on two calls in a row (the full-size slice
at R = 16, then a smaller slice at R = 3, whose call reuses the scratch the
first one left), and a slice whose workspace exceeds the scratch is refused
before anything is launched."""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import synthetic as syn
from helpers import dev, host, packed

pytestmark = pytest.mark.gpu


def _both(x, gate, up, down):
    R, I = x.shape[0], gate.N
    y0 = torch.empty((R, gate.K), dtype=torch.float32, device="cuda")
    h0 = torch.empty((R, I), dtype=torch.int16, device="cuda")
    ev.verify_mlp_w4(x, gate, up, down, y=y0, h=h0)
    y1 = torch.full_like(y0, float("nan"))
    h1 = torch.full_like(h0, -1)
    ev.verify_mlp_w4_noalloc(x, gate, up, down, y1, h=h1)
    torch.cuda.synchronize()
    return host(y0), host(h0), host(y1), host(h1)


def test_noalloc_matches_workspace_entry_point_twice():
    print("noalloc: full-size slice R=16, then H=2048 I=6144 R=3", flush=True)
    d = syn.mlp()
    G = d["G"]
    mats = [packed(d[m], G) for m in ("gate", "up", "down")]
    y0, h0, y1, h1 = _both(dev(d["x"]), *mats)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(h0, h1)
    del mats
    torch.cuda.empty_cache()
    g = np.random.default_rng(77)
    H, I, G = 2048, 6144, 64
    mats = [packed(syn.w4_matrix(g, n, k, G), G) for n, k in ((I, H), (I, H), (H, I))]
    x = dev(syn.activations(g, 3, H))
    y0, h0, y1, h1 = _both(x, *mats)
    assert np.array_equal(y0.view(np.uint32), y1.view(np.uint32))
    assert np.array_equal(h0, h1)


def test_noalloc_refuses_a_slice_beyond_the_scratch():
    H, I, G = 256, 1 << 20, 64
    assert ev.verify_mlp_w4_workspace(H, I, G) > (32 << 20)
    blob = torch.zeros(16, dtype=torch.uint8, device="cuda")
    gate = ev.PackedW4(blob, I, H, G)
    up = ev.PackedW4(blob, I, H, G)
    down = ev.PackedW4(blob, H, I, G)
    x = torch.zeros((1, H), dtype=torch.int16, device="cuda")
    y = torch.zeros((1, H), dtype=torch.float32, device="cuda")
    with pytest.raises(ev.EvError) as e:
        ev.verify_mlp_w4_noalloc(x, gate, up, down, y)
    assert e.value.code == ev.EV_EWORKSPACE
    torch.cuda.synchronize()
    assert not y.any()
