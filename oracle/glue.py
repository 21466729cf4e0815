"""The element-wise glue either side of a decoder layer's projections, in
fp64 with the fp16 roundings of an fp16 model (test infrastructure only).

The zoo's Qwen3-VL page (Architecture paragraph and the size table) describes
the decoder these projections belong to: a Qwen3 text decoder whose MLP is
SwiGLU (gate and up projections, an activation, the down projection).  The
pages do not print the activation or the normalisation; the readings taken
here are the plainest ones for a Qwen3 decoder run in fp16:

* RMSNorm, the input of the q|k|v and gate|up projections: for one token,
  r = 1 / sqrt(mean_k x_k^2 + eps), n_k = fp16(x_k r), out_k = fp16(g_k n_k)
  with g the layer's fp16 norm weight.  The statistic is taken in high
  precision; the normalised value is stored as fp16 before the weight is
  applied.  eps is a parameter (the workloads use 1e-6; the pages give none).
* SwiGLU, the input of the down projection: h_k = fp16(fp16(silu(a_k)) b_k),
  a = the gate projection's fp16 output, b = the up projection's, and
  silu(a) = a / (1 + exp(-a)).

Every value here is computed in fp64 and rounded to fp16 (nearest, ties to
even) exactly where the readings above store an fp16 value.

Parity unpinned by the pages: they fix neither formula, the epsilon, nor the
rounding points.  The pins tie this module to the mathematics (hand-derived
values, torch's rms_norm, scipy's logistic, exact invariants), not to the
pages.
"""
from __future__ import annotations

import numpy as np


def _fp16(v: np.ndarray) -> np.ndarray:
    """Round fp64 values to fp16, nearest with ties to even (numpy's cast)."""
    return np.asarray(v, np.float64).astype(np.float16)


def rms_inverse(x: np.ndarray, eps: float) -> np.ndarray:
    """r = 1 / sqrt(mean(x^2) + eps) over the last axis, in fp64."""
    x64 = np.asarray(x).astype(np.float64)
    ms = np.mean(x64 * x64, axis=-1, keepdims=True)
    return 1.0 / np.sqrt(ms + eps)


def rmsnorm_fp16(x: np.ndarray, gamma: np.ndarray, eps: float) -> np.ndarray:
    """RMSNorm of fp16 tokens x ([K] or [M, K]) with fp16 weight gamma [K]:
    fp16(gamma * fp16(x * r)), r from ``rms_inverse``.  Returns fp16."""
    x64 = np.asarray(x).astype(np.float64)
    n16 = _fp16(x64 * rms_inverse(x64, eps))
    # gamma * n is a product of two fp16 values: exact in fp64, rounded once.
    return _fp16(np.asarray(gamma).astype(np.float64) * n16.astype(np.float64))


def silu(a: np.ndarray) -> np.ndarray:
    """silu(a) = a / (1 + exp(-a)) in fp64 (exp overflow gives -0 or 0)."""
    a64 = np.asarray(a).astype(np.float64)
    with np.errstate(over="ignore"):
        return a64 / (1.0 + np.exp(-a64))


def silu_fp16(a: np.ndarray) -> np.ndarray:
    """The stored activation of fp16 gate outputs: fp16(silu(a))."""
    return _fp16(silu(a))


def glu_fp16(a: np.ndarray, b: np.ndarray) -> np.ndarray:
    """The gating product of two fp16 arrays, stored as fp16: fp16(a * b)
    (the product of two fp16 values is exact in fp64, so this rounds once)."""
    return _fp16(np.asarray(a).astype(np.float64) * np.asarray(b).astype(np.float64))


def swiglu_fp16(gate: np.ndarray, up: np.ndarray) -> np.ndarray:
    """h = fp16(fp16(silu(gate)) * up) element-wise for fp16 gate and up of
    the same shape.  Returns fp16."""
    return glu_fp16(silu_fp16(gate), up)


def _two_blocks(x: np.ndarray):
    x = np.asarray(x)
    if x.ndim == 1:
        half = x.shape[0] // 2
        return x[:half], x[half:]
    x = x.reshape(2, -1, x.shape[-1])
    return x[0], x[1]


def apply_prologue(kind: str, x: np.ndarray, gamma=None, eps: float = 0.0) -> np.ndarray:
    """The fp16 input a projection multiplies, built from what it is given.

    kind "none": x itself.  "rmsnorm": ``rmsnorm_fp16(x, gamma, eps)``.
    "swiglu": x holds the gate outputs of every token followed by the up
    outputs of every token ([2K] for one token, [2, M, K] or [2M, K] for M
    tokens); returns ``swiglu_fp16(gate, up)`` of shape [K] or [M, K].
    "glu": the same two blocks, already activated first block:
    ``glu_fp16(a, b)``."""
    if kind == "none":
        return np.asarray(x)
    if kind == "rmsnorm":
        return rmsnorm_fp16(x, gamma, eps)
    if kind == "swiglu":
        return swiglu_fp16(*_two_blocks(x))
    if kind == "glu":
        return glu_fp16(*_two_blocks(x))
    raise ValueError(kind)
