"""Weight rows that reach the quantizers' rarely taken branches: the code
clamps and signed zeros.  Generators only; none of the method's arithmetic.

int8 b32 clamps need an fp16-subnormal scale that rounds well below a/127:
a block whose absmax is a = 127 f 2^-24 stores the scale round(f) 2^-24, so
for f = 1.4 the largest quotient is 127 * 1.4 = 177.8.

INT4 g64 clamps need the fp16 min to land far from the true min compared
with the scale: a group c + d u (u in [0, 1]) whose offset c sits `off`
above (or below) an fp16 grid point has |mn - fp16(mn)| ~ off while the
scale is d / 15.
"""
from __future__ import annotations

import numpy as np

# f in a = 127 f 2^-24: stored scales 1, 1, 2, 1 and 0 (x 2^-24).  The first
# three clamp codes on both signs, 0.6 stays in range, 0.4 underflows to a
# zero scale.
INT8_SUBNORMAL_F = (1.4, 1.49, 2.4, 0.6, 0.4)


def int8_clamp_rows(k: int, seed: int = 3) -> np.ndarray:
    """[len(INT8_SUBNORMAL_F) + 1, k] fp32 rows of 32-blocks with subnormal
    scales; each block holds +a and -a and values spread in between.  The
    last row alternates the block kinds along K."""
    rng = np.random.default_rng(seed)
    kinds = INT8_SUBNORMAL_F
    rows = np.zeros((len(kinds) + 1, k), np.float32)
    for r in range(len(kinds) + 1):
        for b in range(k // 32):
            f = kinds[r] if r < len(kinds) else kinds[b % len(kinds)]
            a = np.float32(127 * f * 2.0 ** -24)
            blk = (rng.uniform(-1.0, 1.0, 32) * a).astype(np.float32)
            blk[rng.integers(0, 32)] = a
            j = rng.integers(0, 32)
            while blk[j] == a:
                j = rng.integers(0, 32)
            blk[j] = -a
            rows[r, 32 * b:32 * b + 32] = blk
    return rows


def _fp16_grid_point(v: float) -> float:
    return float(np.float16(v))


def int4_clamp_rows(k: int, seed: int = 4) -> np.ndarray:
    """[6, k] fp32 rows of 64-groups c + d u, u ~ U[0, 1]: c = g + off next
    to an fp16 grid point g near 0.3 (or -0.7, 3.1), so that fp16(mn) = g.
    off > 0 puts every quotient above 15 when d is small (clamp high),
    off < 0 below 0 (clamp low); a larger d clamps only some codes."""
    rng = np.random.default_rng(seed)
    cases = [  # (grid base, offset as a fraction of the fp16 step there, spread d)
        (0.3, 0.45, 5e-5), (0.3, -0.45, 5e-5), (-0.7, 0.4, 3e-5),
        (-0.7, -0.4, 3e-5), (3.1, 0.3, 1e-2), (3.1, -0.3, 1e-2)]
    rows = np.zeros((len(cases), k), np.float32)
    for r, (base, frac, d) in enumerate(cases):
        g = _fp16_grid_point(base)
        step = float(np.spacing(np.float16(abs(g))))
        c = g + frac * step
        for gi in range(k // 64):
            u = rng.uniform(0.0, 1.0, 64)
            u[rng.integers(0, 64)] = 0.0
            grp = (c + d * u).astype(np.float32)
            rows[r, 64 * gi:64 * gi + 64] = grp
    return rows


def signed_zero_rows(k: int) -> np.ndarray:
    """[8, k] fp32 rows whose 64-groups (and so 32-blocks) mix +0 and -0:
    all +0; all -0; +0 then -0; -0 then +0; positives with one -0; positives
    with one +0; positives with both zeros; negatives with both zeros (a
    negative min, zeros irrelevant)."""
    rows = np.zeros((8, k), np.float32)
    rng = np.random.default_rng(5)
    nz = np.float32(-0.0)
    for gi in range(k // 64):
        s = slice(64 * gi, 64 * gi + 64)
        rows[0, s] = 0.0
        rows[1, s] = nz
        rows[2, s] = np.where(np.arange(64) % 2 == 0, np.float32(0.0), nz)
        rows[3, s] = np.where(np.arange(64) % 2 == 0, nz, np.float32(0.0))
        pos = (np.abs(rng.standard_normal(64)) * 0.02 + 1e-3).astype(np.float32)
        rows[4, s] = pos
        rows[4, 64 * gi + (gi * 7) % 64] = nz
        rows[5, s] = pos
        rows[5, 64 * gi + (gi * 5) % 64] = 0.0
        rows[6, s] = pos
        rows[6, 64 * gi + (gi * 3) % 64] = 0.0
        rows[6, 64 * gi + (gi * 3 + 11) % 64] = nz
        rows[7, s] = -pos
        rows[7, 64 * gi + (gi * 3) % 64] = 0.0
        rows[7, 64 * gi + (gi * 3 + 11) % 64] = nz
    return rows
