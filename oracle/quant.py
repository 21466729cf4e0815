"""Canonical quantizers and dequantizers (numpy; test infrastructure only).

int8 b32 (symmetric absmax, block of 32 along K)
    Source: Qwen3-VL 4B/8B Core AI cards, Files table ("int8 per-block-32 body
    + untied absmax int8 head"); zoo Qwen3-VL page, Measured paragraph (int8hu
    = int8lin per-block-32 body + untied absmax int8 head); zoo Qwen3.8-27B
    page, Numerics paragraph ("absmax symmetric per-block-32 head rule",
    clipping not used).  The same rule serves body and head.

    Per block of 32 weights w (fp32) of one row:
      a   = max |w|                         exact in fp32
      s32 = fl32(a / 127)                   IEEE fp32 division, RNE
      s   = fp16_RNE(s32)                   the stored scale
      q   = 0                               if s == 0
          = clamp(rint(fl32(w / s)), -127, 127)   otherwise (ties to even)
      w^  = q * s                           (exact in fp64)

    Readings (the pages give only the names): divisor 127, code -128 unused;
    the quotient uses the STORED fp16 scale so codes and dequantization agree;
    rounding is half-to-even; an all-zero block has scale 0 and codes 0;
    non-finite input or a scale beyond fp16 range is refused.  The clamp to
    +-127 acts only when the stored scale rounded below a/127 by more than
    the half step it leaves, which happens for fp16-subnormal scales
    (a < 127 * 2^-14): e.g. a = 127 * 1.4 * 2^-24 stores s = 2^-24 and
    |w| / s reaches 177.8.

int4 g64 (affine min/max, group of 64 along K)
    Source: CoreML-LLM handoff page, Architecture paragraph ("INT4
    per-grouped-channel (group_size 64, matching the MLX *-4bit builds)").
    The affine form is the workload definition, not the pages' (parity
    unpinned by the pages).

    Per group of 64 weights w (fp32):
      mn, mx = min w, max w                 exact; IEEE 754-2019 minimum and
                                            maximum, which order -0 below +0
      s = fp16_RNE(fl32(fl32(mx - mn) / 15)),  m = fp16_RNE(mn)
      q = 0                                 if s == 0
        = clamp(rint(fl32(fl32(w - m) / s)), 0, 15)
      w^ = m + q * s                        (exact in fp64)
    Canonical packing: uint32 word j of a row holds codes 8j..8j+7, code 8j+i
    in bits [4i, 4i+4) (low nibble = lowest k).

    Readings: a group whose least value is zero stores the min -0 (bits
    0x8000) when any of its zeros is -0, else +0; the sign of a zero max never
    reaches a stored bit (mx - mn is +0 or exactly |mn|).  The clamp to 0..15
    acts when fp16 rounding of the min or the scale moves a code past the
    ends, e.g. a group 0.3 + 1e-5 u, whose range gives s ~ 3e-6 while
    |mn - m| reaches 1.2e-4.

fp16 (unquantized head)
    Source: zoo Qwen3-VL page, Measured table, "2B int8lin (tied fp16 head)"
    row (int8 per-block-32 body with the head kept in fp16, against the
    int8hu row's int8 head).
      w16 = fp16_RNE(w)                     round to nearest, ties to even
      w^  = w16                             (exact in fp64)
    Non-finite input, or a value that rounds beyond the fp16 range, is
    refused.  K must be a multiple of 32 (the tiled layout's block).
"""
from __future__ import annotations

import numpy as np

BLOCK8 = 32
GROUP4 = 64
BLOCK16 = 32
QMAX8 = 127
QMAX4 = 15


def _clamp_codes(qf: np.ndarray, lo: int, hi: int) -> np.ndarray:
    """Clamp rounded quotients to the code range [lo, hi]."""
    return np.clip(qf, lo, hi)


def _group_min_max(groups: np.ndarray):
    """Per group (last axis): IEEE 754-2019 minimum and maximum, which order
    -0 below +0 whatever order the zeros come in."""
    mn = np.min(groups, axis=-1)
    mx = np.max(groups, axis=-1)
    zero = groups == 0
    neg_zero = np.any(zero & np.signbit(groups), axis=-1)
    pos_zero = np.any(zero & ~np.signbit(groups), axis=-1)
    mn = np.where(mn == 0, np.where(neg_zero, np.float32(-0.0), np.float32(0.0)), mn)
    mx = np.where(mx == 0, np.where(pos_zero, np.float32(0.0), np.float32(-0.0)), mx)
    return mn.astype(np.float32), mx.astype(np.float32)


def _check_input(w: np.ndarray, mult: int) -> np.ndarray:
    w = np.asarray(w)
    if w.dtype != np.float32:
        raise TypeError("weights must be float32")
    if w.ndim != 2:
        raise ValueError("weights must be [N, K]")
    if w.shape[1] % mult:
        raise ValueError(f"K={w.shape[1]} is not a multiple of {mult}")
    if not np.all(np.isfinite(w)):
        raise ValueError("non-finite weight")
    return w


def quantize_int8_b32(w: np.ndarray):
    """fp32 [N, K] -> (codes int8 [N, K], scales fp16 [N, K/32])."""
    w = _check_input(w, BLOCK8)
    n, k = w.shape
    blocks = w.reshape(n, k // BLOCK8, BLOCK8)
    a = np.max(np.abs(blocks), axis=2) if k else np.zeros((n, 0), np.float32)
    s32 = (a / np.float32(QMAX8)).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
    if np.any(np.isinf(s16)):
        raise ValueError("scale overflows fp16")
    sf = s16.astype(np.float32)[:, :, None]
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (blocks / sf).astype(np.float32)
    qf = np.rint(quot)
    qf = np.where(sf == 0, np.float32(0), qf)
    q = _clamp_codes(qf, -QMAX8, QMAX8).astype(np.int8)
    return q.reshape(n, k), s16


def dequantize_int8_b32(codes: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """(int8 [N, K], fp16 [N, K/32]) -> fp64 [N, K], w^ = q * s."""
    return codes.astype(np.float64) * np.repeat(scales.astype(np.float64), BLOCK8, axis=1)


def quantize_int4_g64(w: np.ndarray):
    """fp32 [N, K] -> (codes uint8 [N, K] in 0..15, scales fp16 [N, K/64],
    mins fp16 [N, K/64])."""
    w = _check_input(w, GROUP4)
    n, k = w.shape
    groups = w.reshape(n, k // GROUP4, GROUP4)
    if k:
        mn, mx = _group_min_max(groups)
    else:
        mn = mx = np.zeros((n, 0), np.float32)
    rng = (mx - mn).astype(np.float32)
    s32 = (rng / np.float32(QMAX4)).astype(np.float32)
    with np.errstate(over="ignore"):
        s16 = s32.astype(np.float16)
        m16 = mn.astype(np.float16)
    if np.any(np.isinf(s16)) or np.any(np.isinf(m16)):
        raise ValueError("scale or min overflows fp16")
    sf = s16.astype(np.float32)[:, :, None]
    mf = m16.astype(np.float32)[:, :, None]
    shifted = (groups - mf).astype(np.float32)
    with np.errstate(divide="ignore", invalid="ignore"):
        quot = (shifted / sf).astype(np.float32)
    qf = np.rint(quot)
    qf = np.where(sf == 0, np.float32(0), qf)
    q = _clamp_codes(qf, 0, QMAX4).astype(np.uint8)
    return q.reshape(n, k), s16, m16


def dequantize_int4_g64(codes: np.ndarray, scales: np.ndarray, mins: np.ndarray) -> np.ndarray:
    """(uint8 codes [N, K], fp16 [N, K/64] x2) -> fp64 [N, K], w^ = m + q * s."""
    s = np.repeat(scales.astype(np.float64), GROUP4, axis=1)
    m = np.repeat(mins.astype(np.float64), GROUP4, axis=1)
    return m + codes.astype(np.float64) * s


def quantize_fp16(w: np.ndarray):
    """fp32 [N, K] -> (fp16 [N, K],) rounded to nearest, ties to even."""
    w = _check_input(w, BLOCK16)
    with np.errstate(over="ignore"):
        h = w.astype(np.float16)
    if np.any(np.isinf(h)):
        raise ValueError("weight overflows fp16")
    return (h,)


def dequantize_fp16(h: np.ndarray) -> np.ndarray:
    """fp16 [N, K] -> fp64 [N, K] (exact)."""
    return h.astype(np.float64)


def pack_nibbles(codes: np.ndarray) -> np.ndarray:
    """uint8 codes [N, K] (0..15) -> canonical uint32 words [N, K/8];
    code 8j+i sits in bits [4i, 4i+4) of word j."""
    n, k = codes.shape
    c = codes.astype(np.uint32).reshape(n, k // 8, 8)
    words = np.zeros((n, k // 8), np.uint32)
    for i in range(8):
        words |= c[:, :, i] << np.uint32(4 * i)
    return words


def unpack_nibbles(words: np.ndarray) -> np.ndarray:
    """Inverse of ``pack_nibbles``."""
    n, kw = words.shape
    out = np.empty((n, kw, 8), np.uint8)
    for i in range(8):
        out[:, :, i] = (words >> np.uint32(4 * i)) & np.uint32(0xF)
    return out.reshape(n, kw * 8)
