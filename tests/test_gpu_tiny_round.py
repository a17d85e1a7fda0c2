"""The tiny verify round end to end on the GPU: one W4 linear (K=256 -> N=512,
G=64) on R in {1,2,4} lanes, the keyed sampler over V=512 (T=0.8, top-k 20,
top-p 0.95, seed 42, positions 0..R-1), and the accept rule with drafts chosen
from the oracle's samples so that exactly two are accepted (fewer when R < 2).
"""
import numpy as np
import pytest

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from helpers import NEAR_TIE, ROW_REL_TOL, dev, host, packed, row_rel_err

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("R", [1, 2, 4])
def test_tiny_round(R):
    t = syn.tiny()
    x = t["x"][:R]
    G, V = t["G"], t["N"]
    w = (t["q"], t["s"], t["b"])
    pos = np.arange(R, dtype=np.int64)
    # oracle: logits (fp64 -> fp32), samples, drafts with exactly min(2, R) accepted
    rl = oracle.w4_linear(x, *w, G, out_f32=True)
    rt, rg, _, _ = oracle.sample_rows(rl, pos, t["T"], t["top_k"], t["top_p"], t["seed"])
    draft = rt.copy()
    if R > 2:
        draft[2] = (rt[2] + 1) % V
    ra, rn = oracle.accept(rt, draft)
    assert ra == min(2, R)
    # GPU
    y = ev.verify_linear_w4(dev(x), packed(w, G))
    assert np.all(row_rel_err(host(y), rl) <= ROW_REL_TOL)
    tok = ev.keyed_sample(y, dev(pos), t["T"], t["top_k"], t["top_p"], t["seed"])
    ht = host(tok)
    near = rg < NEAR_TIE
    assert np.all((ht == rt) | near), (ht, rt, rg)
    a, n = ev.accept_prefix(tok, dev(draft))
    if not near.any():
        assert (int(host(a)[0]), int(host(n)[0])) == (ra, rn)
