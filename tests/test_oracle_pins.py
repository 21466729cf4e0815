"""Pins of the CPU oracle against things other than itself: IEEE rounding
written out from the format definitions, brute-force argmin on tiny inputs,
closed forms, invariants, exact rational products, and the bundle sizes the
pages print.  Chosen so that a dropped term, a wrong sign or index, or a
transposed operand in the oracle fails at least one of them."""
import math
from fractions import Fraction

import numpy as np
import pytest

import synthetic_inputs as si
from oracle import layout, linear, quant
from tests import exact_fp as X
from tests import hard_weights

RNG = np.random.default_rng(12345)


# ---------------------------------------------------------------- IEEE steps

def _fp16_edge_values():
    vals = [0.0, 1.0, -1.0, 65504.0, 65519.99, 65520.0, 65536.0, 6.103515625e-05,
            5.960464477539063e-08, 2.98e-08, 2.9802322387695312e-08, 1e-9, 0.1, 1 / 3]
    # exact midpoints between neighbouring fp16 values (ties) and near-ties
    for base in (1.0, 0.0009765625, 3.0517578125e-05, 1024.0, 6.0e-08):
        h = np.float16(base)
        nxt = np.nextafter(h, np.float16(np.inf))
        mid = (float(h) + float(nxt)) / 2
        vals += [mid, np.nextafter(np.float32(mid), np.float32(0)).item(),
                 np.nextafter(np.float32(mid), np.float32(1e9)).item()]
    vals += list(RNG.standard_normal(300) * 0.02) + list(RNG.standard_normal(100) * 1e-5)
    return [float(np.float32(v)) for v in vals]


def test_numpy_fp16_cast_is_ieee_rne():
    for v in _fp16_edge_values():
        for s in (1, -1):
            with np.errstate(over="ignore"):
                got = float(np.float32(s * v).astype(np.float16))
            want = X.fp16(Fraction(s * v))
            assert got == want or (math.isinf(got) and math.isinf(want) and got == want), (v, got, want)


def test_numpy_fp32_division_is_ieee_rne():
    a = np.abs(RNG.standard_normal(2000).astype(np.float32) * np.float32(0.06))
    for v in a[:400]:
        got = float(np.float32(v) / np.float32(127))
        assert got == X.fp32(Fraction(float(v)) / 127)
    w = RNG.standard_normal(400).astype(np.float32) * np.float32(0.02)
    for v in w:
        s = float(np.float16(0.000431))
        got = float(np.float32(v) / np.float32(s))
        assert got == X.fp32(Fraction(float(v)) / Fraction(s))


# ---------------------------------------------------------------- int8 b32

def _near_tie(t: Fraction, rel: float) -> bool:
    frac = t - math.floor(t)
    return abs(frac - Fraction(1, 2)) <= abs(t) * Fraction(rel)


def _brute_int8(wrow):
    """Reference for one block: scale from the definition's two roundings,
    codes by exhaustive search of the nearest of 255 levels."""
    a = max(abs(Fraction(float(v))) for v in wrow)
    s = X.fp16(X.fp32(a / 127))
    if s == 0:
        return [0] * len(wrow), s, [False] * len(wrow)
    S = Fraction(s)
    codes, ambiguous = [], []
    for v in wrow:
        W = Fraction(float(v))
        best = min(range(-127, 128), key=lambda q: (abs(W - q * S), q % 2))
        codes.append(best)
        ambiguous.append(_near_tie(W / S, 2.0 ** -24))
    return codes, s, ambiguous


@pytest.mark.parametrize("scale", [0.02, 1e-3, 3.0])
def test_int8_brute_force_argmin(scale):
    w = (RNG.standard_normal((6, 96)) * scale).astype(np.float32)
    q, s = quant.quantize_int8_b32(w)
    for n in range(6):
        for b in range(3):
            blk = w[n, 32 * b:32 * b + 32]
            codes, s_ref, amb = _brute_int8(blk)
            assert float(s[n, b]) == s_ref
            for i in range(32):
                if amb[i]:
                    assert abs(int(q[n, 32 * b + i]) - codes[i]) <= 1
                else:
                    assert int(q[n, 32 * b + i]) == codes[i], (n, b, i)


def test_int8_exact_ties_round_to_even():
    # absmax 127 * 2^-7 makes the scale exactly 2^-7; then w = (c + 1/2) 2^-7 is a tie
    s = 2.0 ** -7
    blk = np.zeros(32, np.float32)
    blk[0] = 127 * s
    halves = [0.5, 1.5, 2.5, -0.5, -1.5, -2.5, 10.5, 11.5, -126.5, 125.5]
    blk[1:1 + len(halves)] = np.array(halves, np.float32) * np.float32(s)
    q, sc = quant.quantize_int8_b32(blk[None, :])
    assert float(sc[0, 0]) == s
    want = [X.round_half_even(Fraction(h).limit_denominator(4)) for h in halves]
    assert [int(v) for v in q[0, 1:1 + len(halves)]] == want
    assert want == [0, 2, 2, 0, -2, -2, 10, 12, -126, 126]


def test_int8_scale_closed_forms():
    # a = 127 v for an fp16 value v is exact in fp32, so the stored scale is v
    for v in [2.0 ** -10, 0.000431, 0.0215, 1.0, 7.25, 511.5]:
        v16 = float(np.float16(v))
        blk = np.zeros((1, 32), np.float32)
        blk[0, 5] = np.float32(-127 * v16)
        blk[0, 6] = np.float32(0.5 * v16)
        q, s = quant.quantize_int8_b32(blk)
        assert float(s[0, 0]) == v16
        assert int(q[0, 5]) == -127


def _roundtrip_ok(w, w_hat, s_rep):
    err = np.abs(w.astype(np.float64) - w_hat)
    return np.all(err <= s_rep / 2 * (1 + 2.0 ** -16))


def test_int8_roundtrip_bound_and_no_clamp():
    w = si.weights(7, 64, 512)
    q, s = quant.quantize_int8_b32(w)
    w_hat = quant.dequantize_int8_b32(q, s)
    s_rep = np.repeat(s.astype(np.float64), 32, axis=1)
    assert _roundtrip_ok(w, w_hat, s_rep)
    # every block attains |q| = 127 exactly at its absmax element (normal scales)
    assert np.all(np.abs(q.reshape(64, 16, 32).astype(int)).max(axis=2) == 127)


def test_int8_sign_symmetry_and_pow2_scaling():
    w = si.weights(8, 32, 256)
    q, s = quant.quantize_int8_b32(w)
    qn, sn = quant.quantize_int8_b32(-w)
    assert np.array_equal(qn, -q) and np.array_equal(sn, s)
    for e in (-1, 1, 3, 6):
        # the invariance holds while every scale stays an fp16 normal number
        assert s.astype(np.float64).min() * 2.0 ** e >= 2.0 ** -14
        qe, se = quant.quantize_int8_b32((w * np.float32(2.0 ** e)).astype(np.float32))
        assert np.array_equal(qe, q)
        assert np.array_equal(se.astype(np.float64), s.astype(np.float64) * 2.0 ** e)


def test_int8_idempotent():
    w = si.weights(9, 32, 256)
    q, s = quant.quantize_int8_b32(w)
    w_hat = quant.dequantize_int8_b32(q, s).astype(np.float32)
    q2, s2 = quant.quantize_int8_b32(w_hat)
    assert np.array_equal(q2, q) and np.array_equal(s2, s)


def test_int8_zero_blocks():
    w = si.weights(10, 4, 128)
    w[1, 32:64] = 0
    w[3, :] = 0
    q, s = quant.quantize_int8_b32(w)
    assert float(s[1, 1]) == 0 and not q[1, 32:64].any()
    assert not s[3].any() and not q[3].any()
    x = si.activations(11, 1, 128)[0]
    y = linear.ref_linear("int8_b32", (q, s), x)
    assert y[3] == 0.0


def test_int8_refuses_bad_input():
    w = np.zeros((2, 64), np.float32)
    w[0, 3] = np.nan
    with pytest.raises(ValueError):
        quant.quantize_int8_b32(w)
    w[0, 3] = 127 * 70000.0
    with pytest.raises(ValueError):
        quant.quantize_int8_b32(w)
    with pytest.raises(ValueError):
        quant.quantize_int8_b32(np.zeros((2, 48), np.float32))


def _int8_mismatches(w, q, s):
    bad = []
    for n in range(w.shape[0]):
        for b in range(w.shape[1] // 32):
            codes, s_ref, amb = _brute_int8(w[n, 32 * b:32 * b + 32])
            if float(s[n, b]) != s_ref:
                bad.append((n, b, "scale"))
            for i in range(32):
                got = int(q[n, 32 * b + i])
                if (abs(got - codes[i]) > 1) if amb[i] else (got != codes[i]):
                    bad.append((n, b, i))
    return bad


def _int8_clamp_events(w):
    """(high, low) counts of weights whose exact quotient by the stored scale
    lies beyond +-127.5: those the clamp decides."""
    hi = lo = 0
    for n in range(w.shape[0]):
        for b in range(w.shape[1] // 32):
            blk = w[n, 32 * b:32 * b + 32]
            s = Fraction(X.fp16(X.fp32(max(abs(Fraction(float(v))) for v in blk) / 127)))
            if s == 0:
                continue
            for v in blk:
                t = Fraction(float(v)) / s
                hi += t > Fraction(255, 2)
                lo += t < -Fraction(255, 2)
    return hi, lo


def test_int8_clamp_subnormal_scales_brute_force():
    """Blocks with fp16-subnormal scales that round well below a/127 reach
    the +-127 clamp on both signs; codes must still be the nearest of the
    255 levels (the clamp picks the end level)."""
    w = hard_weights.int8_clamp_rows(256)
    hi, lo = _int8_clamp_events(w)
    assert hi > 0 and lo > 0, (hi, lo)
    q, s = quant.quantize_int8_b32(w)
    assert _int8_mismatches(w, q, s) == []
    assert int(q.min()) == -127 and int(q.max()) == 127


# ---------------------------------------------------------------- int4 g64

def _brute_int4(blk):
    """Reference for one group: scale and min from the definition's
    roundings, codes by exhaustive search of the nearest of 16 levels."""
    mn, mx = Fraction(float(blk.min())), Fraction(float(blk.max()))
    s_ref = X.fp16(X.fp32(Fraction(X.fp32(mx - mn)) / 15))
    m_ref = X.fp16(mn)
    S, M = Fraction(s_ref), Fraction(m_ref)
    codes, ambiguous = [], []
    for v in blk:
        W = Fraction(float(v))
        if S == 0:
            codes.append(0)
            ambiguous.append(False)
            continue
        codes.append(min(range(16), key=lambda c: (abs(W - (M + c * S)), c % 2)))
        ambiguous.append(_near_tie((W - M) / S, 2.0 ** -22))
    return codes, s_ref, m_ref, ambiguous


def _int4_mismatches(w, q, s, m):
    bad = []
    for n in range(w.shape[0]):
        for g in range(w.shape[1] // 64):
            blk = w[n, 64 * g:64 * g + 64]
            codes, s_ref, m_ref, amb = _brute_int4(blk)
            if float(s[n, g]) != s_ref or float(m[n, g]) != m_ref:
                bad.append((n, g, "scale/min"))
            for i in range(64):
                got = int(q[n, 64 * g + i])
                if (abs(got - codes[i]) > 1) if amb[i] else (got != codes[i]):
                    bad.append((n, g, i))
    return bad


def test_int4_brute_force_argmin():
    w = si.weights(20, 4, 128)
    q, s, m = quant.quantize_int4_g64(w)
    assert _int4_mismatches(w, q, s, m) == []


def _int4_clamp_events(w):
    hi = lo = 0
    for n in range(w.shape[0]):
        for g in range(w.shape[1] // 64):
            blk = w[n, 64 * g:64 * g + 64]
            _, s_ref, m_ref, _ = _brute_int4(blk)
            if s_ref == 0:
                continue
            for v in blk:
                t = (Fraction(float(v)) - Fraction(m_ref)) / Fraction(s_ref)
                hi += t > Fraction(31, 2)
                lo += t < -Fraction(1, 2)
    return hi, lo


def test_int4_clamp_brute_force():
    """Groups whose fp16 min lands far from the true min compared with the
    scale reach both clamps (all codes of a group, or only its ends)."""
    w = hard_weights.int4_clamp_rows(256)
    hi, lo = _int4_clamp_events(w)
    assert hi > 0 and lo > 0, (hi, lo)
    q, s, m = quant.quantize_int4_g64(w)
    assert _int4_mismatches(w, q, s, m) == []
    assert int(q.min()) == 0 and int(q.max()) == 15


# Planted mistakes in the oracle's clamp: each must fail a pin above.
_CLAMP_MUTANTS = {
    "no clamp": lambda qf, lo, hi: qf,
    "int8 floor -128": lambda qf, lo, hi: np.clip(qf, lo - 1 if lo < 0 else lo, hi),
    "int4 clamp to 255, masked": lambda qf, lo, hi: (np.clip(qf, lo, 255) % 16 if hi == 15
                                                    else np.clip(qf, lo, hi)),
    "int4 floor -1": lambda qf, lo, hi: np.clip(qf, -1 if hi == 15 else lo, hi),
    "int8 ceiling 126": lambda qf, lo, hi: np.clip(qf, lo, hi - 1 if hi == 127 else hi),
}


@pytest.mark.parametrize("name", sorted(_CLAMP_MUTANTS))
def test_clamp_mutants_fail_the_pins(monkeypatch, name):
    monkeypatch.setattr(quant, "_clamp_codes", _CLAMP_MUTANTS[name])
    w8 = hard_weights.int8_clamp_rows(128)
    w4 = hard_weights.int4_clamp_rows(128)
    with np.errstate(invalid="ignore", over="ignore"):
        q8, s8 = quant.quantize_int8_b32(w8)
        q4, s4, m4 = quant.quantize_int4_g64(w4)
    caught = bool(_int8_mismatches(w8, q8, s8)) or bool(_int4_mismatches(w4, q4, s4, m4))
    assert caught, f"planted mistake '{name}' passes every clamp pin"


def _ieee2019_min(vals):
    """IEEE 754-2019 minimum over a list: the least value, -0 below +0."""
    return min(vals, key=lambda v: (v, 0 if (v == 0 and math.copysign(1.0, v) < 0) else 1))


def test_int4_signed_zero_min():
    """A group's stored min follows IEEE 754-2019 minimum: -0 (bits 0x8000)
    when the least value is zero and any zero is -0, whatever the order;
    zero groups have a zero scale and zero codes."""
    w = hard_weights.signed_zero_rows(128)
    q, s, m = quant.quantize_int4_g64(w)
    mbits = m.view(np.uint16)
    for n in range(w.shape[0]):
        for g in range(2):
            blk = [float(v) for v in w[n, 64 * g:64 * g + 64]]
            want = np.float16(_ieee2019_min(blk)).view(np.uint16)
            assert int(mbits[n, g]) == int(want), (n, g, hex(int(mbits[n, g])), hex(int(want)))
    assert [int(b) for b in mbits[:4, 0]] == [0x0000, 0x8000, 0x8000, 0x8000]
    assert int(mbits[4, 0]) == 0x8000 and int(mbits[5, 0]) == 0 and int(mbits[6, 0]) == 0x8000
    assert not s[:4].view(np.uint16).any() and not q[:4].any()
    assert _int4_mismatches(w, q, s, m) == []


def test_int4_order_dependent_min_fails_the_pin(monkeypatch):
    """A min that keeps whichever zero comes first (plain np.min) is caught."""
    def first_zero(groups):
        return groups.min(axis=-1), groups.max(axis=-1)
    monkeypatch.setattr(quant, "_group_min_max", first_zero)
    with pytest.raises(AssertionError):
        test_int4_signed_zero_min()


def test_int4_roundtrip_and_degenerate():
    w = si.weights(21, 32, 256)
    w[5, 64:128] = np.float32(0.0123)
    w[6, :64] = 0
    q, s, m = quant.quantize_int4_g64(w)
    w_hat = quant.dequantize_int4_g64(q, s, m)
    s_rep = np.repeat(s.astype(np.float64), 64, axis=1)
    err = np.abs(w.astype(np.float64) - w_hat)
    live = s_rep > 0
    assert np.all(err[live] <= s_rep[live] * (0.5 + 2.0 ** -18))
    # a constant group has zero scale, zero codes and dequantizes to fp16(value)
    assert float(s[5, 1]) == 0 and not q[5, 64:128].any()
    assert np.all(w_hat[5, 64:128] == float(np.float16(0.0123)))
    assert float(s[6, 0]) == 0 and float(m[6, 0]) == 0 and not w_hat[6, :64].any()


def test_int4_pow2_scaling_and_idempotence():
    w = si.weights(22, 16, 256)
    q, s, m = quant.quantize_int4_g64(w)
    q2, s2, m2 = quant.quantize_int4_g64((w * np.float32(4.0)).astype(np.float32))
    assert np.array_equal(q2, q)
    assert np.array_equal(s2.astype(np.float64), 4 * s.astype(np.float64))
    assert np.array_equal(m2.astype(np.float64), 4 * m.astype(np.float64))
    w_hat = quant.dequantize_int4_g64(q, s, m).astype(np.float32)
    q3, s3, m3 = quant.quantize_int4_g64(w_hat)
    assert np.array_equal(q3, q) and np.array_equal(s3, s) and np.array_equal(m3, m)


def test_nibble_packing():
    codes = np.array([[1, 2, 3, 4, 5, 6, 7, 8, 15, 0, 0, 0, 0, 0, 0, 9]], np.uint8)
    words = quant.pack_nibbles(codes)
    assert words[0, 0] == 0x87654321 and words[0, 1] == 0x9000000F
    c = RNG.integers(0, 16, (5, 64)).astype(np.uint8)
    assert np.array_equal(quant.unpack_nibbles(quant.pack_nibbles(c)), c)


# ---------------------------------------------------------------- layout

@pytest.mark.parametrize("n,k", [(16, 256), (37, 544), (5, 32), (48, 1024)])
def test_int8_layout_bijection_and_size(n, k):
    q = RNG.integers(-127, 128, (n, k)).astype(np.int8)
    s = (RNG.standard_normal((n, k // 32)) * 1e-3).astype(np.float16)
    blob = layout.tile_int8_b32(q, s)
    assert blob.size == layout.packed_bytes("int8_b32", n, k)
    q2, s2 = layout.untile_int8_b32(blob, n, k)
    assert np.array_equal(q2, q) and np.array_equal(s2.view(np.uint16), s.view(np.uint16))
    if n % 16 == 0 and k % 256 == 0:
        assert blob.size * 32 == n * k * 34


@pytest.mark.parametrize("n,k", [(16, 256), (37, 576), (3, 64), (32, 1024)])
def test_int4_layout_bijection_and_size(n, k):
    q = RNG.integers(0, 16, (n, k)).astype(np.uint8)
    s = (RNG.standard_normal((n, k // 64)) * 1e-3).astype(np.float16)
    m = (RNG.standard_normal((n, k // 64)) * 1e-2).astype(np.float16)
    blob = layout.tile_int4_g64(q, s, m)
    assert blob.size == layout.packed_bytes("int4_g64", n, k)
    q2, s2, m2 = layout.untile_int4_g64(blob, n, k)
    assert np.array_equal(q2, q)
    assert np.array_equal(s2.view(np.uint16), s.view(np.uint16))
    assert np.array_equal(m2.view(np.uint16), m.view(np.uint16))
    if n % 16 == 0 and k % 256 == 0:
        assert blob.size * 64 == n * k * 36


def _golden_rows(name):
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", name)
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            yield [int(t, 0) for t in line.split()]


def test_int8_layout_hand_offsets():
    n, k = 32, 512
    # codes encode their own position so every byte names its source
    q = np.zeros((n, k), np.int8)
    s = np.zeros((n, k // 32), np.float16)
    for off, row, col in _golden_rows("layout_int8_offsets.txt"):
        q[:] = 0
        q[row, col] = 77
        blob = layout.tile_int8_b32(q, s)
        hits = np.flatnonzero(blob == 77)
        assert list(hits) == [off], (off, row, col, hits)
    # scale bytes: scale (row, block) lands at the hand-derived offset
    q[:] = 0
    s[17, 9] = np.float16(-2.0)      # bits 0xC000
    blob = layout.tile_int8_b32(q, s)
    # row 17 -> r=1, rho=1; block 9 -> j=1, beta=1: tile (1,1) = (1*2+1)*4352
    off = 3 * 4352 + 4096 + 16 * 1 + 2 * 1
    assert blob[off] == 0x00 and blob[off + 1] == 0xC0
    assert np.count_nonzero(blob) == 1


def test_fp16_layout_hand_offsets():
    n, k = 32, 512
    h = np.zeros((n, k), np.float16)
    for off, row, col in _golden_rows("layout_fp16_offsets.txt"):
        h[:] = 0
        h[row, col] = np.float16(-2.0)          # bits 0xC000: one nonzero byte
        blob = layout.tile_fp16(h)
        hits = np.flatnonzero(blob)
        assert list(hits) == [off + 1] and blob[off + 1] == 0xC0, (off, row, col, hits)


def _fp16_grid():
    """Every finite fp16 value as (bits, float64), in increasing value order."""
    bits = np.arange(0, 1 << 16, dtype=np.uint32).astype(np.uint16)
    vals = bits.view(np.float16).astype(np.float64)
    ok = np.isfinite(vals)
    bits, vals = bits[ok], vals[ok]
    order = np.argsort(vals, kind="stable")
    bits, vals = bits[order], vals[order]
    keep = np.ones(len(vals), bool)             # drop -0 (same value as +0)
    keep[1:] = vals[1:] != vals[:-1]
    return bits[keep], vals[keep]


def _rne_fp16_brute(x: float, grid_bits, grid_vals):
    """Round x to the nearest finite fp16 value, ties to the even bit pattern,
    by searching the whole fp16 grid (None if x rounds beyond the largest)."""
    i = int(np.searchsorted(grid_vals, x))
    cand = [j for j in (i - 1, i) if 0 <= j < len(grid_vals)]
    best = min(cand, key=lambda j: abs(grid_vals[j] - x))
    ties = [j for j in cand if abs(grid_vals[j] - x) == abs(grid_vals[best] - x)]
    if len(ties) == 2:
        best = ties[0] if int(grid_bits[ties[0]]) % 2 == 0 else ties[1]
    top = grid_vals[-1]                         # 65504
    if abs(x) >= top + (top - grid_vals[-2]) / 2:
        return None                             # at or past the midpoint to 65536
    return best


def test_fp16_rounding_brute_force():
    """The fp16 head's conversion is round-to-nearest-even onto the fp16 grid:
    random values across the whole exponent range, exact midpoints between
    neighbours (ties), subnormals and the values around the largest finite."""
    gb, gv = _fp16_grid()
    rng = np.random.default_rng(16)
    xs = list((rng.standard_normal(600) * np.exp2(rng.integers(-26, 16, 600))).astype(np.float32))
    picks = rng.integers(1, len(gv) - 1, 400)
    xs += [np.float32((gv[i] + gv[i + 1]) / 2) for i in picks]          # exact midpoints (fit in fp32)
    xs += [np.float32(v) for v in (0.0, 5.96e-8, 2.98e-8, 2.99e-8, 6.1e-5, 65504.0, 65519.0, -65519.0)]
    for x in xs:
        j = _rne_fp16_brute(float(x), gb, gv)
        assert j is not None
        (h,) = quant.quantize_fp16(np.full((1, 32), x, np.float32))
        want = np.uint16(gb[j])
        got = h.view(np.uint16)[0, 0]
        # +0 and -0 are the same value; compare values there, bits elsewhere
        if gv[j] == 0.0:
            assert h[0, 0] == 0.0
        else:
            assert got == want, (x, hex(got), hex(want))
    for bad in (65520.0, -65520.0, 1e6, np.inf, np.nan):
        with pytest.raises(ValueError):
            quant.quantize_fp16(np.full((1, 32), bad, np.float32))


def test_fp16_round_trip_bound():
    """|w - w^| <= half the fp16 spacing at w^ (normal range), and w^ exactly
    representable values convert to themselves."""
    rng = np.random.default_rng(17)
    w = (rng.standard_normal((8, 256)) * 0.02).astype(np.float32)
    (h,) = quant.quantize_fp16(w)
    wh = quant.dequantize_fp16(h)
    spacing = np.abs(np.spacing(h.astype(np.float16)).astype(np.float64))
    assert np.all(np.abs(w.astype(np.float64) - wh) <= spacing / 2)
    (h2,) = quant.quantize_fp16(h.astype(np.float32))
    assert np.array_equal(h2.view(np.uint16), h.view(np.uint16))


def test_fp16_layout_bijection_and_size():
    for n, k in ((16, 256), (37, 544), (1, 32), (48, 1024)):
        rng = np.random.default_rng(n * 1000 + k)
        (h,) = quant.quantize_fp16(rng.standard_normal((n, k)).astype(np.float32))
        blob = layout.tile_fp16(h)
        assert blob.size == layout.packed_bytes("fp16", n, k)
        (h2,) = layout.untile_fp16(blob, n, k)
        assert np.array_equal(h2.view(np.uint16), h.view(np.uint16))
        if n % 16 == 0 and k % 256 == 0:
            assert blob.size == n * k * 2


def test_int4_layout_hand_offsets():
    n, k = 32, 512
    s = np.zeros((n, k // 64), np.float16)
    m = np.zeros((n, k // 64), np.float16)
    q = np.zeros((n, k), np.uint8)
    for off, nib, row, col in _golden_rows("layout_int4_offsets.txt"):
        q[:] = 0
        q[row, col] = 0xA
        blob = layout.tile_int4_g64(q, s, m)
        hits = np.flatnonzero(blob)
        assert list(hits) == [off], (off, row, col, hits)
        assert blob[off] == (0xA << (4 * nib)), (off, nib, row, col, blob[off])
    q[:] = 0
    m[2, 5] = np.float16(1.0)        # bits 0x3C00 ; row 2 -> r0 rho2; group 5 -> j1, slot 1
    blob = layout.tile_int4_g64(q, s, m)
    off = 1 * 2304 + 2048 + 16 * 2 + 8 + 2 * 1
    assert blob[off] == 0x00 and blob[off + 1] == 0x3C and np.count_nonzero(blob) == 1


# ---------------------------------------------------------------- products

def test_single_nonzero_block_closed_form():
    # only row 2, block 1 is nonzero: y = s * sum_{i<32} q_i x_{32+i} on row 2, 0 elsewhere
    w = np.zeros((4, 64), np.float32)
    vals = np.arange(-16, 16, dtype=np.float32) * np.float32(2.0 ** -8)
    vals[0] = np.float32(127 * 2.0 ** -8)           # absmax -> scale exactly 2^-8
    w[2, 32:64] = vals
    q, s = quant.quantize_int8_b32(w)
    assert float(s[2, 1]) == 2.0 ** -8
    x = (np.arange(64) % 7 - 3).astype(np.float16)
    y = linear.ref_linear("int8_b32", (q, s), x)
    codes = [127] + list(range(-15, 16))
    want = sum(c * int(x[32 + i]) for i, c in enumerate(codes)) * 2.0 ** -8
    assert y[2] == want and y[0] == 0 and y[1] == 0 and y[3] == 0
    # the transposed product must not agree (guards a swapped operand)
    assert y.shape == (4,)


def test_int4_single_group_closed_form():
    w = np.zeros((2, 128), np.float32)
    # values m + c*s with s = 2^-6, m = -2^-3 for c = 0..15 (then repeated)
    c = np.tile(np.arange(16), 4)
    w[1, 64:] = (np.float32(-0.125) + c.astype(np.float32) * np.float32(2.0 ** -6))
    q, s, m = quant.quantize_int4_g64(w)
    assert float(s[1, 1]) == 2.0 ** -6 and float(m[1, 1]) == -0.125
    assert np.array_equal(q[1, 64:], c.astype(np.uint8))
    x = (np.arange(128) % 5 - 2).astype(np.float16)
    y = linear.ref_linear("int4_g64", (q, s, m), x)
    want = sum((-0.125 + int(ci) * 2.0 ** -6) * int(x[64 + i]) for i, ci in enumerate(c))
    assert y[1] == want and y[0] == 0


@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
def test_exact_rational_dot(fmt):
    w = si.weights(30, 5, 128)
    parts = quant.quantize_int8_b32(w) if fmt == "int8_b32" else quant.quantize_int4_g64(w)
    x = si.activations(31, 1, 128)[0]
    y = linear.ref_linear(fmt, parts, x)
    w_hat = linear.dequantize(fmt, parts)
    for n in range(5):
        terms = [Fraction(float(w_hat[n, k])) * Fraction(float(x[k])) for k in range(128)]
        exact = sum(terms)
        bound = 128 * 2.0 ** -52 * float(sum(abs(t) for t in terms))
        assert abs(Fraction(float(y[n])) - exact) <= Fraction(bound)


def test_linearity_and_rows():
    w = si.weights(32, 40, 256)
    parts = quant.quantize_int8_b32(w)
    X16 = si.activations(33, 3, 256)
    Y = linear.ref_linear("int8_b32", parts, X16)
    assert Y.shape == (3, 40)
    for mrow in range(3):
        y = linear.ref_linear("int8_b32", parts, X16[mrow])
        assert np.array_equal(y, Y[mrow])
        y4 = linear.ref_linear("int8_b32", parts, (X16[mrow].astype(np.float32) * 4).astype(np.float16))
        assert np.array_equal(y4, 4 * y)
    rows = [0, 17, 39]
    assert np.array_equal(linear.ref_linear_rows("int8_b32", parts, X16[0], rows), Y[0, rows])


def test_stack_chaining_rounds_to_fp16():
    w1 = si.weights(34, 64, 64)
    w2 = si.weights(35, 32, 64)
    p1, p2 = quant.quantize_int8_b32(w1), quant.quantize_int8_b32(w2)
    x = si.activations(36, 1, 64)[0]
    outs = linear.ref_stack([{"fmt": "int8_b32", "parts": p1, "x": x},
                             {"fmt": "int8_b32", "parts": p2, "x_from": 0}])
    y1 = linear.ref_linear("int8_b32", p1, x)
    assert np.array_equal(outs[0], y1)
    assert np.array_equal(outs[1], linear.ref_linear("int8_b32", p2, y1.astype(np.float16)))


# ---------------------------------------------------------------- page pins

def test_bundle_sizes_match_pages():
    """The int8hu bundles' printed sizes pin one byte plus one 16-bit scale per
    32 weights: linear stack in the tiled int8 format + an fp16 embedding
    table reproduce every size the pages print.  The printed value is rounded
    to 0.1, and the bundles also carry a tokenizer and metadata (the cards'
    Files tables say so) that are not counted here, worth at most ~0.02 GiB:
    so the counted bytes must lie in [page - 0.07, page + 0.05) GiB.  A
    16-bit scale per 64 weights, a 32-bit scale per 32, or no scales at all
    each miss the 8B size by more than 0.2 GiB."""
    for name, layers, hidden, q_heads, mlp, head_kind, page_gb in _golden_sizes():
        d = si.Decoder(name, layers, hidden, q_heads, mlp)
        body = sum(layout.packed_bytes("int8_b32", n, k)
                   for gname, ms in d.groups() if gname != "head" for _, n, k in ms)
        embed = d.vocab * hidden * 2
        head = layout.packed_bytes("int8_b32", d.vocab, hidden) if head_kind == "int8" else 0
        total_gib = (body + embed + head) / 2 ** 30
        assert page_gb - 0.07 <= total_gib < page_gb + 0.05, (name, total_gib, page_gb)


def _golden_sizes():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "bundle_sizes.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if not line:
            continue
        t = line.split()
        yield t[0], int(t[1]), int(t[2]), int(t[3]), int(t[4]), t[5], float(t[6])


# ---------------------------------------------------------------- glue (RMSNorm, SwiGLU)

def _golden_glue():
    import os
    path = os.path.join(os.path.dirname(__file__), "golden", "glue_hand_values.txt")
    for line in open(path):
        line = line.split("#")[0].strip()
        if line:
            yield line


def test_glue_hand_values():
    """Hand-derived values, including two double-rounding cases (gamma applied
    to the stored fp16 normalised value; up applied to the stored fp16 silu)
    and the tie cases, which a single rounding or another rounding mode fails."""
    from oracle import glue
    seen = {"rmsnorm": 0, "swiglu": 0}
    for line in _golden_glue():
        kind, rest = line.split(None, 1)
        seen[kind] += 1
        if kind == "rmsnorm":
            head, gam, want = rest.split("|")
            eps, *xs = head.split()
            x = np.array([float(v) for v in xs], np.float16)
            g = np.array([float(v) for v in gam.split()], np.float16)
            got = glue.rmsnorm_fp16(x, g, float(eps))
            assert got.dtype == np.float16
            assert np.array_equal(got.astype(np.float64), [float(v) for v in want.split()]), line
        else:
            a, b, want = (float(v) for v in rest.split())
            got = glue.swiglu_fp16(np.array([a], np.float16), np.array([b], np.float16))
            assert got.dtype == np.float16 and float(got[0]) == want, (line, float(got[0]))
            assert math.copysign(1.0, float(got[0])) == math.copysign(1.0, want), line
    assert seen["rmsnorm"] >= 4 and seen["swiglu"] >= 6


def test_rmsnorm_matches_library_rms_norm():
    """torch's fp64 rms_norm (weight-free) rounded to fp16 is the oracle's
    normalised value; with gamma the oracle applies it to that fp16 value."""
    import torch
    from oracle import glue
    x = si.activations(71, 4, 1024)
    g = (RNG.standard_normal(1024) * 0.3 + 1.0).astype(np.float16)
    for eps in (1e-6, 1e-2):
        n_lib = torch.nn.functional.rms_norm(torch.from_numpy(x.astype(np.float64)), (1024,),
                                             eps=eps).numpy().astype(np.float16)
        ones = np.ones(1024, np.float16)
        n_or = glue.rmsnorm_fp16(x, ones, eps)
        # the two fp64 statistics may differ in their last bit; that moves an
        # fp16 rounding at most one step, and only next to a midpoint
        diff = np.abs(n_or.astype(np.float64) - n_lib.astype(np.float64))
        ulp = np.spacing(np.abs(n_lib).astype(np.float16)).astype(np.float64)
        assert np.all(diff <= ulp) and np.mean(diff == 0) > 0.999
        full = glue.rmsnorm_fp16(x, g, eps)
        assert np.array_equal(full, (g.astype(np.float64) * n_or.astype(np.float64)).astype(np.float16))


def test_rmsnorm_invariants():
    """Per-token statistic (tokens do not mix), exact power-of-two scale
    invariance when eps = 0, and the mean over K (not K - 1, not the sum)."""
    from oracle import glue
    x = si.activations(72, 3, 256)
    g = np.full(256, 1.0, np.float16)
    both = glue.rmsnorm_fp16(x, g, 0.0)
    for t in range(3):
        assert np.array_equal(both[t], glue.rmsnorm_fp16(x[t], g, 0.0))
    x4 = (x.astype(np.float64) * 4).astype(np.float16)
    assert np.array_equal(glue.rmsnorm_fp16(x4, g, 0.0), both)
    # a token of K equal values v: mean(x^2) = v^2 exactly, so n = 1
    for k in (2, 32, 256):
        v = np.full(k, 0.375, np.float16)
        assert np.all(glue.rmsnorm_fp16(v, np.ones(k, np.float16), 0.0) == 1.0)
    assert np.all(np.isfinite(glue.rmsnorm_fp16(np.zeros(64, np.float16), np.ones(64, np.float16), 1e-6)))


def test_silu_identities_and_library():
    """silu(a) - silu(-a) = a, silu(a) = a * expit(a) (scipy's logistic), and
    fp16(silu) with up = 1 is the SwiGLU output."""
    from scipy.special import expit
    from oracle import glue
    a = np.concatenate([RNG.standard_normal(2000) * 4, np.linspace(-30, 30, 601)])
    s = glue.silu(a)
    assert np.allclose(s - glue.silu(-a), a, rtol=0, atol=1e-12 * np.maximum(1, np.abs(a)).max())
    assert np.allclose(s, a * expit(a), rtol=1e-14, atol=1e-300)
    a16 = a.astype(np.float16)
    ones = np.ones_like(a16)
    assert np.array_equal(glue.swiglu_fp16(a16, ones), glue.silu(a16).astype(np.float16))
    # up = 2^j scales exactly (no overflow or subnormal results here)
    big = a16[np.abs(glue.silu(a16)) > 1e-3]
    for j in (-3, 1, 4):
        u = np.full(big.shape, 2.0 ** j, np.float16)
        assert np.array_equal(glue.swiglu_fp16(big, u).astype(np.float64),
                              glue.swiglu_fp16(big, np.ones_like(big)).astype(np.float64) * 2.0 ** j)


def test_prologue_layouts_and_stack():
    """SwiGLU input layouts (one token: gate then up; M tokens: all gates then
    all ups), and ref_stack feeding a SwiGLU op from a [gate, up] pair."""
    from oracle import glue
    a = si.activations(73, 3, 64)
    b = si.activations(74, 3, 64)
    want = glue.swiglu_fp16(a, b)
    assert np.array_equal(glue.apply_prologue("swiglu", np.concatenate([a, b], 0)), want)
    assert np.array_equal(glue.apply_prologue("swiglu", np.concatenate([a[1], b[1]])), want[1])
    w_g, w_u, w_d = si.weights(75, 64, 128), si.weights(76, 64, 128), si.weights(77, 32, 64)
    pg, pu, pd = (quant.quantize_int8_b32(w) for w in (w_g, w_u, w_d))
    x = si.activations(78, 1, 128)[0]
    gam = (RNG.standard_normal(128) * 0.2 + 1).astype(np.float16)
    outs = linear.ref_stack([
        {"fmt": "int8_b32", "parts": pg, "x": x, "prologue": ("rmsnorm", gam, 1e-6)},
        {"fmt": "int8_b32", "parts": pu, "x": x, "prologue": ("rmsnorm", gam, 1e-6)},
        {"fmt": "int8_b32", "parts": pd, "x_from": [0, 1], "prologue": ("swiglu", None, 0.0)}])
    xn = glue.rmsnorm_fp16(x, gam, 1e-6)
    g_ref = linear.ref_linear("int8_b32", pg, xn)
    u_ref = linear.ref_linear("int8_b32", pu, xn)
    assert np.array_equal(outs[0], g_ref) and np.array_equal(outs[1], u_ref)
    h = glue.swiglu_fp16(g_ref.astype(np.float16), u_ref.astype(np.float16))
    assert np.array_equal(outs[2], linear.ref_linear("int8_b32", pd, h))


def test_glu_product_rounds_once_to_even():
    """fp16(a * b): 3 * (1 + 2^-10) = 1537.5 * 2^-9, a tie, goes to the even
    1538 * 2^-9; (1 + 2^-10)^2 = 1 + 2^-9 + 2^-20 rounds down to 1 + 2^-9;
    65504 * 2 overflows to inf (the IEEE result)."""
    from oracle import glue
    a = np.array([3.0, 1.0009765625, 65504.0, -0.5], np.float16)
    b = np.array([1.0009765625, 1.0009765625, 2.0, 0.25], np.float16)
    with np.errstate(over="ignore"):
        got = glue.glu_fp16(a, b).astype(np.float64)
    assert got[0] == 1538 * 2.0 ** -9 and got[1] == 1 + 2.0 ** -9
    assert np.isinf(got[2]) and got[3] == -0.125
    x = np.concatenate([a, b])
    with np.errstate(over="ignore"):
        assert np.array_equal(glue.apply_prologue("glu", x), glue.glu_fp16(a, b))
