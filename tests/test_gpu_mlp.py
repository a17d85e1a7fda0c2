"""GPU parity of the dense SiLU-gated MLP verify slice.

Small shapes: per-row relative error of y <= 2e-3, and h (bf16) within one bf16
ulp of the oracle's h (the two sides round slightly different fp32 values).
Every row of an R-lane call is bit-identical to the row called alone.
Full size (5120 -> 17408 -> 5120, G = 64, R = 16): y on sampled columns, with
the oracle computing the whole gate/up stage and the sampled down columns.
"""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from helpers import ROW_REL_TOL, dev, host, row_rel_err, weights_dev

pytestmark = pytest.mark.gpu


def _mlp(x, gate, up, down, G):
    R = x.shape[0]
    I = gate[0].shape[0]
    h = torch.empty((R, I), dtype=torch.int16, device="cuda")
    y = ev.verify_mlp_w4(dev(x), weights_dev(gate), weights_dev(up), weights_dev(down), G, h=h)
    return host(y), host(h).view(np.uint16)


@pytest.mark.parametrize("H,I,G", [(256, 384, 64), (256, 96, 32), (512, 1024, 32), (2048, 768, 32)])
def test_small_mlp_parity_and_row_exactness(H, I, G):
    g = np.random.default_rng(H + I + G)
    gate = syn.w4_matrix(g, I, H, G)
    up = syn.w4_matrix(g, I, H, G)
    down = syn.w4_matrix(g, H, I, G)
    x = syn.activations(g, 16, H)
    ry, _, _, rh = oracle.mlp(x, gate, up, down, G)
    y, h = _mlp(x, gate, up, down, G)
    assert np.all(row_rel_err(y, ry) <= ROW_REL_TOL)
    hv, rv = syn.bf16_values(h).astype(np.float64), syn.bf16_values(rh).astype(np.float64)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(rv), 1e-30))) - 7)
    assert np.all(np.abs(hv - rv) <= ulp)
    assert np.mean(h != rh) < 1e-3
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
    assert np.mean(h != rh) < 1e-3
    cols = np.unique(np.concatenate([np.arange(0, d["H"], 53), [d["H"] - 1]]))
    q, s, b = d["down"]
    ry = oracle.w4_linear(rh, q[cols], s[cols], b[cols], G)
    err = row_rel_err(y[:, cols], ry)
    assert np.all(err <= ROW_REL_TOL), err
    torch.cuda.empty_cache()
