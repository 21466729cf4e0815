"""Acceptance checks shared by the GPU parity tests.

Bound per output vector (one projection, one token row), against the oracle's
unrounded fp64 result y_ref over the dequantized weights w^:
  max_n |y[n] - y_ref[n]| <= 2e-3 * ||x||_2 * max_k |w^[n, k]|
  ||y - y_ref||_2 <= 1e-3 * ||y_ref||_2
Where the bound is zero (an all-zero weight row) the output must be exactly 0.
"""
from __future__ import annotations

import numpy as np

MAX_ERR_COEF = 2e-3
REL_L2 = 1e-3


def check_vector(y_gpu, y_ref, row_max, x, what=""):
    y = np.asarray(y_gpu, dtype=np.float64)
    y_ref = np.asarray(y_ref, dtype=np.float64)
    assert y.shape == y_ref.shape, (what, y.shape, y_ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    xn = float(np.linalg.norm(np.asarray(x, dtype=np.float64)))
    err = np.abs(y - y_ref)
    bound = MAX_ERR_COEF * xn * np.asarray(row_max, dtype=np.float64)
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (f"{what}: {bad.size} outputs over the bound; first rows {bad[:8]}, "
                           f"err {err[bad[:4]]}, bound {bound[bad[:4]]}")
    ref_norm = float(np.linalg.norm(y_ref))
    if ref_norm == 0.0:
        assert float(np.linalg.norm(y)) == 0.0, f"{what}: expected all-zero output"
    else:
        rel = float(np.linalg.norm(y - y_ref)) / ref_norm
        assert rel <= REL_L2, f"{what}: relative L2 error {rel:.3e} > {REL_L2}"
    return float(err.max(initial=0.0))
