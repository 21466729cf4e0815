"""The decode-time quantized linear layer in fp64: dequantize, then multiply
(test infrastructure only).

The pages state the workload, not the kernel: every decode step streams all
quantized weights once and forms y = W^ x for each projection (Core AI 4B/8B
cards, Measured paragraph: "Decode is bandwidth-bound"); the zoo's Qwen3.8-27B
page adds a static S=16 prefill chunk beside the S=1 decode function (vision
path section), i.e. Y = X W^T with 16 token rows.

Everything here is plain fp64 numpy: the dequantized matrix is formed
explicitly and multiplied with a BLAS product.  Results are not rounded.
"""
from __future__ import annotations

import numpy as np

from . import glue, quant

ROW_CHUNK = 16384   # rows dequantized at a time, to bound memory


def dequantize(fmt: str, parts) -> np.ndarray:
    if fmt == "int8_b32":
        return quant.dequantize_int8_b32(*parts)
    if fmt == "int4_g64":
        return quant.dequantize_int4_g64(*parts)
    if fmt == "fp16":
        return quant.dequantize_fp16(*parts)
    raise ValueError(fmt)


def _slice_parts(parts, r0, r1):
    return tuple(p[r0:r1] for p in parts)


def ref_linear(fmt: str, parts, x: np.ndarray) -> np.ndarray:
    """y[n] = sum_k w^[n, k] x[k] in fp64, for x of shape [K] (M=1) or [M, K].

    Returns [N] or [M, N]."""
    x64 = np.asarray(x).astype(np.float64)
    n = parts[0].shape[0]
    outs = []
    for r0 in range(0, n, ROW_CHUNK):
        w_hat = dequantize(fmt, _slice_parts(parts, r0, min(n, r0 + ROW_CHUNK)))
        outs.append(x64 @ w_hat.T)
    if not outs:
        return np.zeros(x64.shape[:-1] + (0,), np.float64)
    return np.concatenate(outs, axis=-1)


def ref_linear_rows(fmt: str, parts, x: np.ndarray, rows) -> np.ndarray:
    """``ref_linear`` restricted to the given output rows ([len(rows)] or [M, len(rows)])."""
    rows = np.asarray(rows)
    sub = tuple(p[rows] for p in parts)
    return ref_linear(fmt, sub, x)


def row_max_abs(fmt: str, parts) -> np.ndarray:
    """max_k |w^[n, k]| per row (for the acceptance bound)."""
    n = parts[0].shape[0]
    out = np.empty(n, np.float64)
    for r0 in range(0, n, ROW_CHUNK):
        r1 = min(n, r0 + ROW_CHUNK)
        w_hat = dequantize(fmt, _slice_parts(parts, r0, r1))
        out[r0:r1] = np.abs(w_hat).max(axis=1) if w_hat.shape[1] else 0.0
    return out


def ref_stack(ops):
    """Decode-step linear stack, op by op in the given order.

    ``ops`` is a list of dicts with keys ``fmt``, ``parts`` (canonical
    quantized arrays), ``x`` (fp16 activation, [K] or [M, K]) or ``x_from``
    (index of an earlier op whose output, rounded to fp16, is this op's
    input; for a SwiGLU prologue a pair [gate op, up op], whose outputs are
    joined gate first), and optionally ``prologue`` = (kind, gamma, eps), the
    glue of ``glue.apply_prologue`` that turns the given activation into the
    multiplied one.  Returns the list of fp64 outputs.  An op fed by an earlier
    op sees that op's output rounded to fp16, as a stored fp16 activation is.
    """
    outs = []
    for op in ops:
        if "x_from" in op:
            src = op["x_from"]
            if isinstance(src, (list, tuple)):
                x = np.concatenate([outs[i].astype(np.float16).reshape(1, -1) if outs[i].ndim == 1
                                    else outs[i].astype(np.float16) for i in src], axis=0)
                if outs[src[0]].ndim == 1:
                    x = x.reshape(-1)
            else:
                x = outs[src].astype(np.float16)
        else:
            x = op["x"]
        kind, gamma, eps = op.get("prologue", ("none", None, 0.0))
        x = glue.apply_prologue(kind, x, gamma, eps)
        outs.append(ref_linear(op["fmt"], op["parts"], x))
    return outs
