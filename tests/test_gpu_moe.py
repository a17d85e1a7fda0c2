"""GPU parity of the MoE verify layer (verify_moe_w4) against the oracle.

* routing: expert ids in rank order identical to the oracle's (a selection, no
  arithmetic); renormalised weights within 1e-6;
* y: per-row relative error <= 2e-3 against the oracle (fp64 experts, fp64
  combine in rank order);
* row exactness: every row of an R-lane call is bit-identical to that row
  called alone, and to the same row inside a call with the lanes reversed
  (so a lane sits at another row of its experts' tiles);
* edge cases: all lanes routed alike (one full 16-row group per expert), every
  expert selected (top == E), top = 1, tied router logits (lower id first).
Full size (30B-A3B-like layer: H 2048, 128 experts, top 8, I 768, G 32, R 16)
against the oracle on every row.
"""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from helpers import ROW_REL_TOL, dev, host, row_rel_err

pytestmark = pytest.mark.gpu


def _stack(w, G):
    q, s, b = w
    return ev.w4_pack_stack(dev(q), dev(s), dev(b), G)


class _Layer:
    def __init__(self, gate, up, down, top, G):
        self.gate, self.up, self.down = _stack(gate, G), _stack(up, G), _stack(down, G)
        self.top, self.G = top, G
        self.ws = torch.empty(ev.verify_moe_w4_workspace(self.gate.K, self.gate.N, self.gate.E, top, G),
                              dtype=torch.uint8, device="cuda")

    def __call__(self, x, rho):
        R = x.shape[0]
        ids = torch.empty((R, self.top), dtype=torch.int32, device="cuda")
        w = torch.empty((R, self.top), dtype=torch.float32, device="cuda")
        y = ev.verify_moe_w4(dev(x), dev(rho), self.gate, self.up, self.down, self.top,
                             expert_ids=ids, expert_w=w, ws=self.ws)
        torch.cuda.synchronize()
        return host(y), host(ids), host(w)


def _weights(g, H, I, E, G):
    def stack(rows, cols):
        q, s, b = syn.w4_matrix(g, E * rows, cols, G)
        return q.reshape(E, rows, -1), s.reshape(E, rows, -1), b.reshape(E, rows, -1)
    return stack(I, H), stack(I, H), stack(H, I)


def _check(layer, x, rho, gate, up, down, top, G, exact_rows=True):
    y, ids, w = layer(x, rho)
    ry, rids, rw = oracle.moe(x, rho, top, G, gate, up, down)
    assert np.array_equal(ids, rids)
    assert np.max(np.abs(w - rw)) < 1e-6
    err = row_rel_err(y, ry)
    assert np.all(err <= ROW_REL_TOL), err
    if exact_rows:
        R = x.shape[0]
        for r in range(R):
            y1, _, _ = layer(x[r:r + 1], rho[r:r + 1])
            assert np.array_equal(y1[0].view(np.uint32), y[r].view(np.uint32)), r
        yr, _, _ = layer(x[::-1].copy(), rho[::-1].copy())
        assert np.array_equal(yr[::-1].view(np.uint32), y.view(np.uint32))
    return err


@pytest.mark.parametrize("H,I,E,top,G", [(256, 128, 16, 4, 32), (256, 192, 8, 8, 64),
                                         (512, 256, 32, 1, 32), (384, 96, 24, 3, 32),
                                         (256, 128, 256, 8, 32),  # the most experts and the largest top
                                         (256, 96, 100, 6, 32)])  # experts filling part of the last wave
@pytest.mark.parametrize("R", [1, 5, 16])
def test_small_moe_parity_and_row_exactness(H, I, E, top, G, R):
    g = np.random.default_rng(H * 7 + I + E + top + G)
    gate, up, down = _weights(g, H, I, E, G)
    layer = _Layer(gate, up, down, top, G)
    x = syn.activations(g, R, H)
    rho = g.standard_normal((R, E), dtype=np.float32)
    _check(layer, x, rho, gate, up, down, top, G)


def test_all_lanes_on_the_same_experts_and_ties():
    H, I, E, top, G = 256, 128, 16, 4, 32
    g = np.random.default_rng(77)
    gate, up, down = _weights(g, H, I, E, G)
    layer = _Layer(gate, up, down, top, G)
    x = syn.activations(g, 16, H)
    rho = np.tile(g.standard_normal((1, E), dtype=np.float32), (16, 1))
    _check(layer, x, rho, gate, up, down, top, G)
    # ties: equal logits everywhere but two lanes; -0 and +0 tie too
    rho = np.zeros((16, E), np.float32)
    rho[3, 5] = 1.0
    rho[7, ::2] = -0.0
    y, ids, _ = layer(x, rho)
    ry, rids, _ = oracle.moe(x, rho, top, G, gate, up, down)
    assert np.array_equal(ids, rids)
    assert list(ids[0]) == [0, 1, 2, 3] and list(ids[3]) == [5, 0, 1, 2]
    assert np.all(row_rel_err(y, ry) <= ROW_REL_TOL)


def test_full_size_moe_layer():
    d = syn.moe()
    G, top = d["G"], d["top"]
    layer = _Layer(d["gate"], d["up"], d["down"], top, G)
    err = _check(layer, d["x"], d["rho"], d["gate"], d["up"], d["down"], top, G, exact_rows=False)
    print(f"full-size MoE: max row rel err {err.max():.3e}")
    y, _, _ = layer(d["x"], d["rho"])
    for r in (0, 9, 15):
        y1, _, _ = layer(d["x"][r:r + 1], d["rho"][r:r + 1])
        assert np.array_equal(y1[0].view(np.uint32), y[r].view(np.uint32)), r
