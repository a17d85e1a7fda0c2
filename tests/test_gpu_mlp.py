"""GPU parity of the dense SiLU-gated MLP verify slice.

Small shapes (the split gate/up launch with its SiLU kernel, and one shape wide
enough for the paired launch): per-row relative error of y <= 2e-3, and h (bf16) within one bf16
ulp of the oracle's h plus the first-order effect of the linears' absolute
error (eps = 1e-5 of each row's max |g|, |u|) on silu(g) * u -- near g = 0 or
u = 0 a tiny absolute error in g or u is a large relative error in h.

How many h elements may differ from the oracle's at all: h is a bf16
rounding of silu(g) * u, and an error dh in the product moves the rounding
across a boundary with probability |dh| / ulp(h) (the exact value's place
inside its bf16 interval is spread evenly).  With eps the GPU's measured
largest error of g and u relative to the row's largest value (the linears
called alone), the expected fraction of differing elements is at most
mean(min(1, dh / ulp)), dh the first-order bound above at that eps; the test
allows twice that plus 1e-4.
Every row of an R-lane call is bit-identical to the row called alone.
Full size (5120 -> 17408 -> 5120, G = 64, R = 16): y on sampled columns, with
the oracle computing the whole gate/up stage and the sampled down columns;
and every row of the R = 1, 2, 4, 8 and 16 calls bit-identical (y and h) to
that row called alone.
"""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from helpers import ROW_REL_TOL, dev, host, packed, row_rel_err

pytestmark = pytest.mark.gpu


def _mlp(x, gate, up, down, G):
    R = x.shape[0]
    I = gate[0].shape[0]
    h = torch.empty((R, I), dtype=torch.int16, device="cuda")
    y = ev.verify_mlp_w4(dev(x), packed(gate, G), packed(up, G), packed(down, G), h=h)
    return host(y), host(h).view(np.uint16)


def _h_bound(g, u, eps):
    """First-order bound on |d(silu(g) u)| for errors eps * max|g|, eps * max|u| per row."""
    dg = eps * np.max(np.abs(g), axis=1, keepdims=True)
    du = eps * np.max(np.abs(u), axis=1, keepdims=True)
    sig = 1.0 / (1.0 + np.exp(-g))
    silu = g * sig
    dsilu = sig * (1.0 + g * (1.0 - sig))  # derivative of silu, |.| <= 1.1
    return np.abs(dsilu * u) * dg + np.abs(silu) * du


def _measured_eps(x, gate, up, G, g, u):
    """Largest error of the GPU's gate and up linears (called alone) relative
    to each row's largest oracle value."""
    yg = host(ev.verify_linear_w4(dev(x), packed(gate, G)))
    yu = host(ev.verify_linear_w4(dev(x), packed(up, G)))
    return float(max(row_rel_err(yg, g).max(), row_rel_err(yu, u).max()))


def _check_h(h, rh, x, gate, up, G, eps=1e-5):
    x = x[:h.shape[0]]
    g = oracle.w4_linear(x, *gate, G)
    u = oracle.w4_linear(x, *up, G)
    bound = _h_bound(g, u, eps)
    hv, rv = syn.bf16_values(h).astype(np.float64), syn.bf16_values(rh).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(rv), 1e-38))) - 7)
    diff = np.abs(hv - rv)
    bad = diff > ulp + 2.0 * bound
    if bad.any():
        r, c = np.argwhere(bad)[0]
        raise AssertionError(f"h[{r},{c}]: gpu {hv[r, c]!r} oracle {rv[r, c]!r} g {g[r, c]!r} "
                             f"u {u[r, c]!r} ulp {ulp[r, c]!r} bound {bound[r, c]!r}; "
                             f"{int(bad.sum())} elements")
    _check_h_fraction(h, rh, x, gate, up, G, g, u)


def _check_h_fraction(h, rh, x, gate, up, G, g, u):
    eps = _measured_eps(x, gate, up, G, g, u)
    hx = np.abs(syn.bf16_values(rh).astype(np.float64))
    ulp = np.exp2(np.floor(np.log2(np.maximum(hx, 1e-38))) - 7)
    expected = float(np.mean(np.minimum(1.0, _h_bound(g, u, eps) / ulp)))
    frac = float(np.mean(h != rh))
    print(f"h differs from the oracle's in {frac:.2e} of elements; expected at most "
          f"{expected:.2e} (measured eps {eps:.2e})")
    assert frac <= 2.0 * expected + 1e-4


# (384, 32800, 32): enough gate/up tiles (2050) for the paired launch, with a
# ragged last workgroup and K (3 chunks) ending inside the second half
@pytest.mark.parametrize("H,I,G", [(256, 384, 64), (256, 96, 32), (512, 1024, 32), (2048, 768, 32),
                                   (384, 32800, 32)])
def test_small_mlp_parity_and_row_exactness(H, I, G):
    g = np.random.default_rng(H + I + G)
    gate = syn.w4_matrix(g, I, H, G)
    up = syn.w4_matrix(g, I, H, G)
    down = syn.w4_matrix(g, H, I, G)
    x = syn.activations(g, 16, H)
    ry, _, _, rh = oracle.mlp(x, gate, up, down, G)
    y, h = _mlp(x, gate, up, down, G)
    assert np.all(row_rel_err(y, ry) <= ROW_REL_TOL)
    _check_h(h, rh, x, gate, up, G)
    for r in (0, 9, 15):
        y1, h1 = _mlp(x[r:r + 1], gate, up, down, G)
        assert np.array_equal(y1[0].view(np.uint32), y[r].view(np.uint32))
        assert np.array_equal(h1[0], h[r])
    for R in (2, 5, 8):
        yR, _ = _mlp(x[:R], gate, up, down, G)
        assert np.array_equal(yR.view(np.uint32), y[:R].view(np.uint32))


def test_full_size_mlp_slice_sampled_columns():
    d = syn.mlp()
    G, x = d["G"], d["x"]
    y, h = _mlp(x, d["gate"], d["up"], d["down"], G)
    # oracle: gate/up over all columns, then down on sampled output columns
    g32 = oracle.w4_linear(x, *d["gate"], G, out_f32=True)
    u32 = oracle.w4_linear(x, *d["up"], G, out_f32=True)
    rh = oracle.silu_mul_bf16(g32, u32)
    _check_h_fraction(h, rh, x, d["gate"], d["up"], G, g32.astype(np.float64), u32.astype(np.float64))
    cols = np.unique(np.concatenate([np.arange(0, d["H"], 53), [d["H"] - 1]]))
    q, s, b = d["down"]
    ry = oracle.w4_linear(rh, q[cols], s[cols], b[cols], G)
    err = row_rel_err(y[:, cols], ry)
    assert np.all(err <= ROW_REL_TOL), err
    torch.cuda.empty_cache()


def test_full_size_mlp_slice_rows_bit_exact_at_every_R():
    """The full-size slice (balanced gate/up launch, SiLU segment sum, balanced
    down launch at their real geometry): every row of the R = 2, 4, 8 and 16
    calls equals, bit for bit, that row called alone (R = 1), for y and h."""
    d = syn.mlp()
    G, x = d["G"], d["x"]
    gate, up, down = (packed(d[m], G) for m in ("gate", "up", "down"))
    I = d["I"]
    xd = dev(x)

    def run(rows):
        R = rows.shape[0]
        h = torch.empty((R, I), dtype=torch.int16, device="cuda")
        y = ev.verify_mlp_w4(rows.contiguous(), gate, up, down, h=h)
        return host(y), host(h).view(np.uint16)

    alone = [run(xd[r:r + 1]) for r in range(16)]
    for R in (2, 4, 8, 16):
        y, h = run(xd[:R])
        for r in range(R):
            assert np.array_equal(y[r].view(np.uint32), alone[r][0][0].view(np.uint32)), (R, r)
            assert np.array_equal(h[r], alone[r][1][0]), (R, r)
    # lanes in reverse order: each row still equals itself alone
    y, h = run(torch.flip(xd, [0]))
    for r in range(16):
        assert np.array_equal(y[15 - r].view(np.uint32), alone[r][0][0].view(np.uint32))
    del gate, up, down
    torch.cuda.empty_cache()
