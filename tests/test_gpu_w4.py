"""GPU parity of verify_linear_w4 against the oracle, and row exactness.

* exact-integer and one-hot cases: bit-identical to the oracle;
* random cases at several shapes (ragged N, K with a partial chunk, one and many
  K-splits, balanced runs that cross column blocks, G = 32 and 64): per-row relative error <= 2e-3 (observed ~1e-7);
* every row of an R-lane call is bit-identical to the same row called alone,
  for every R in 1..16, and two runs give the same bits;
* the full-size shapes (MLP gate/up 5120->17408, down 17408->5120, LM head
  5120->151936) in the launch configuration the benchmark uses, on sampled
  output columns the oracle computes one by one;
* the standard-layout entry point (packing inside the call) gives the packed
  entry point's bits.
"""
import numpy as np
import pytest
import torch

import exact_speculative_decoding_amd as ev
import oracle
import synthetic as syn
from helpers import ROW_REL_TOL, dev, host, packed, row_rel_err

pytestmark = pytest.mark.gpu


def _pack(qv):
    qv = qv.astype(np.uint8)
    return (qv[:, 0::2] | (qv[:, 1::2] << 4)).astype(np.uint8)


def _run(x, w, G):
    return host(ev.verify_linear_w4(dev(x), packed(w, G)))


@pytest.mark.parametrize("G", [32, 64])
def test_exact_integer_case_is_bit_identical(G):
    g = np.random.default_rng(21)
    R, K, N = 16, 512, 200
    qv = g.integers(0, 16, (N, K))
    x = syn.bf16_bits(g.integers(-3, 4, (R, K)).astype(np.float32))
    s = syn.fp16_bits(np.full((N, K // G), 2.0 ** -5))
    b = syn.fp16_bits(g.integers(-8, 9, (N, K // G)) * 2.0 ** -10)
    w = (_pack(qv), s, b)
    ref = oracle.w4_linear(x, *w, G, out_f32=True)
    assert np.array_equal(_run(x, w, G), ref)


@pytest.mark.parametrize("G", [32, 64])
def test_one_hot_reads_back_weights_bit_identical(G):
    g = np.random.default_rng(22)
    K, N = 384, 100
    w = syn.w4_matrix(g, N, K, G)
    ks = [0, 1, 7, 8, 31, 32, 63, 64, 127, 128, 200, K - 1, 5, 6, 250, 129]
    x = np.zeros((16, K), np.float32)
    for r, k in enumerate(ks):
        x[r, k] = 1.0
    x = syn.bf16_bits(x)
    assert np.array_equal(_run(x, w, G), oracle.w4_linear(x, *w, G, out_f32=True))


SHAPES = [  # (K, N, G)
    (256, 512, 64),    # the tiny workload
    (96, 33, 32),      # one partial chunk, ragged N
    (320, 40, 32),     # partial last chunk
    (192, 130, 64),    # K % 128 == 64
    (2048, 300, 32),   # several chunks
    (5120, 1000, 64),  # several K-splits
    (4096 + 64, 17, 64),  # one column block summed from 17 workgroups
    (5120, 5000, 64),    # balanced runs of 1-2 superchunks crossing block boundaries
    (4096, 6200, 32),    # the same with group 32, ragged N
    (5248, 2000, 64),    # balanced, an odd number of full chunks (the last superchunk half past K)
]


@pytest.mark.parametrize("K,N,G", SHAPES)
def test_random_parity_with_oracle(K, N, G):
    g = np.random.default_rng(K * 7 + N)
    w = syn.w4_matrix(g, N, K, G)
    x = syn.activations(g, 16, K)
    ref = oracle.w4_linear(x, *w, G)
    for R in (1, 3, 16):
        y = _run(x[:R], w, G)
        err = row_rel_err(y, ref[:R])
        assert np.all(err <= ROW_REL_TOL), err
        # far tighter in practice: fp32 accumulation
        assert np.all(err <= 1e-5), err


@pytest.mark.parametrize("K,N,G", [(256, 512, 64), (320, 40, 32), (5120, 1000, 64), (2048, 300, 32),
                                   (5120, 5000, 64), (4096 + 64, 17, 64), (4096, 6200, 32), (5248, 2000, 64)])
def test_rows_bit_identical_to_single_row_calls(K, N, G):
    g = np.random.default_rng(5 + K + N)
    w = syn.w4_matrix(g, N, K, G)
    x = syn.activations(g, 16, K)
    wp = packed(w, G)
    xd = dev(x)
    alone = np.stack([host(ev.verify_linear_w4(xd[r:r + 1].contiguous(), wp))[0]
                      for r in range(16)])
    for R in range(1, 17):
        y = host(ev.verify_linear_w4(xd[:R].contiguous(), wp))
        assert np.array_equal(y.view(np.uint32), alone[:R].view(np.uint32)), R
    again = host(ev.verify_linear_w4(xd, wp))
    assert np.array_equal(again.view(np.uint32), alone.view(np.uint32))


@pytest.mark.parametrize("name,K,N", [("mlp_gate_up", 5120, 17408), ("mlp_down", 17408, 5120),
                                      ("lm_head", 5120, 151936)])
def test_full_size_sampled_columns(name, K, N):
    G = 64
    g = np.random.default_rng(1002 if name != "lm_head" else 1003)
    q, s, b = syn.w4_matrix(g, N, K, G)
    x = syn.activations(g, 16, K)
    wp = packed((q, s, b), G)
    xd = dev(x)
    y16 = host(ev.verify_linear_w4(xd, wp))
    cols = np.unique(np.concatenate([np.arange(0, N, N // 97), [N - 1, N - 2, 127, 128]]))
    ref = oracle.w4_linear(x, q[cols], s[cols], b[cols], G)
    err = row_rel_err(y16[:, cols], ref)
    assert np.all(err <= ROW_REL_TOL), err
    assert np.all(err <= 1e-5), err
    # rows of the R = 16 pass equal the rows of R = 1 passes, bitwise
    for r in (0, 7, 15):
        y1 = host(ev.verify_linear_w4(xd[r:r + 1].contiguous(), wp))
        assert np.array_equal(y1[0].view(np.uint32), y16[r].view(np.uint32))
    del wp
    torch.cuda.empty_cache()


@pytest.mark.parametrize("K,N", [(16384, 229376), (229376, 16384)])
def test_largest_packed_matrix_sampled_columns(K, N):
    """Packed matrices just under the 2^31-byte limit (G 64): wide (the direct
    launch) and deep (the balanced launch, 896 superchunks a block), so the
    kernels' 32-bit offsets reach the top of their range.  Sampled columns,
    the last ones included, match the oracle; rows equal single-row calls."""
    G = 64
    nbytes = ev.w4_packed_bytes(N, K, G)
    assert 0.98 * 2**31 < nbytes < 2**31
    g = np.random.default_rng(1009 + K)
    q, s, b = syn.w4_matrix(g, N, K, G)
    x = syn.activations(g, 16, K)
    wp = packed((q, s, b), G)
    xd = dev(x)
    y16 = host(ev.verify_linear_w4(xd, wp))
    cols = np.unique(np.concatenate([np.arange(0, N, N // 61), [N - 1, N - 2, N - 16, N - 17, 127, 128]]))
    ref = oracle.w4_linear(x, q[cols], s[cols], b[cols], G)
    del q, s, b
    err = row_rel_err(y16[:, cols], ref)
    assert np.all(err <= ROW_REL_TOL), err
    for r in (0, 15):
        y1 = host(ev.verify_linear_w4(xd[r:r + 1].contiguous(), wp))
        assert np.array_equal(y1[0].view(np.uint32), y16[r].view(np.uint32))
    del wp
    torch.cuda.empty_cache()



@pytest.mark.parametrize("K,N,G", [(256, 512, 64), (384, 200, 32), (5120, 1000, 64), (17408, 64, 64)])
def test_standard_layout_entry_equals_packed(K, N, G):
    g = np.random.default_rng(K + N + G)
    q, sc, bi = syn.w4_matrix(g, N, K, G)
    x = syn.bf16_bits(g.standard_normal((16, K)).astype(np.float32))
    wp = packed((q, sc, bi), G)
    for R in (1, 7, 16):
        ref = host(ev.verify_linear_w4(dev(x[:R]), wp))
        got = host(ev.verify_linear_w4_standard(dev(x[:R]), dev(q), dev(sc), dev(bi), G))
        assert np.array_equal(ref.view(np.int32), got.view(np.int32)), R
