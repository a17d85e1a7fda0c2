"""The packed W4 layout is an exact copy: w4_pack's bytes equal an independent
numpy construction of the layout (16-row tiles by 128-k chunks, chunk-major:
all tiles of chunk 0, then of chunk 1, ...; each tile-chunk holds its codes in
lane order, each dword's 8 codes as even-k then odd-k nibbles, then its
(scale, bias) pairs; zero padding past N and K)."""
import numpy as np
import pytest

import exact_speculative_decoding_amd as ev
import synthetic as syn
from helpers import host, packed

pytestmark = pytest.mark.gpu


def _layout(q, s, b, N, K, G):
    T, NC, GPC = -(-N // 16), -(-K // 128), 128 // G
    Kp, Np = NC * 128, T * 16
    qv = np.zeros((Np, Kp), np.uint8)  # unpacked codes, zero padded
    qv[:N, 0:K:2] = q & 15
    qv[:N, 1:K:2] = q >> 4
    sp = np.zeros((Np, Kp // G), np.uint32)
    sp[:N, :K // G] = s.astype(np.uint32) | (b.astype(np.uint32) << 16)
    out = np.zeros((NC, T, 1024 + 64 * GPC), np.uint8)
    for tile in range(T):
        for c in range(NC):
            blk = np.zeros((64, 4, 8), np.uint8)  # lane, dword t, nibble i
            for L in range(64):
                ln, j = L % 16, L // 16
                for t in range(4):
                    k = 128 * c + 32 * t + 8 * j
                    blk[L, t] = qv[16 * tile + ln, k:k + 8]
            # within a dword, nibbles low to high: q0 q2 q4 q6 q1 q3 q5 q7
            blk = blk[..., [0, 2, 4, 6, 1, 3, 5, 7]]
            codes = (blk[..., 0::2] | (blk[..., 1::2] << 4)).reshape(-1)
            out[c, tile, :1024] = codes
            pairs = sp[16 * tile:16 * tile + 16, c * GPC:(c + 1) * GPC]  # [ln][g]
            out[c, tile, 1024:] = pairs.astype('<u4').view(np.uint8).reshape(-1)
    return out.reshape(-1)


@pytest.mark.parametrize("N,K,G", [(32, 256, 64), (17, 96, 32), (40, 320, 32), (130, 192, 64)])
def test_pack_matches_layout_model(N, K, G):
    g = np.random.default_rng(N * K)
    q, s, b = syn.w4_matrix(g, N, K, G)
    blob = host(packed((q, s, b), G).blob)
    ref = _layout(q, s, b, N, K, G)
    assert blob.size == ev.w4_packed_bytes(N, K, G) == ref.size
    assert np.array_equal(blob, ref)
    if N % 16 == 0 and K % 128 == 0:
        assert blob.size == q.nbytes + s.nbytes + b.nbytes
