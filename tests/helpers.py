"""Shared helpers for the GPU tests: numpy <-> device tensors and the parity
metrics.  Tolerances:
  * logits / linear outputs: per-row max-abs error over the row's max-abs oracle
    value <= 2e-3 (the required bound); the tests also record the observed value.
  * tokens: identical to the oracle's except where the oracle's gap between the
    two best perturbed scores is below 1e-4 (counted, reported).
"""
import numpy as np
import torch

ROW_REL_TOL = 2e-3
NEAR_TIE = 1e-4


def dev(a, dtype=None):
    """numpy array -> device tensor (uint16 bit patterns become int16)."""
    a = np.ascontiguousarray(a)
    if a.dtype == np.uint16:
        a = a.view(np.int16)
    t = torch.from_numpy(a)
    if dtype is not None:
        t = t.to(dtype)
    return t.cuda()


def host(t):
    return t.detach().cpu().numpy()


def row_rel_err(y, ref):
    """max_n |y - ref| / max_n |ref| for each row."""
    y = np.asarray(y, np.float64)
    ref = np.asarray(ref, np.float64)
    den = np.maximum(np.max(np.abs(ref), axis=-1), 1e-30)
    return np.max(np.abs(y - ref), axis=-1) / den


def weights_dev(w):
    q, s, b = w
    return dev(q), dev(s), dev(b)


def packed(w, G):
    """Standard-layout numpy (q, s, b) -> PackedW4 on the device via w4_pack."""
    import exact_speculative_decoding_amd as ev
    q, s, b = weights_dev(w)
    return ev.w4_pack(q, s, b, G)
