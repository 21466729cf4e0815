"""Weight-only quantized decode linear layers for MI355X (gfx950).

Python binding of libqdecode (include/qdecode.h).  Every function here only
marshals arguments: tensors are checked for dtype, device and contiguity, and
their data pointers plus torch's current HIP stream are handed to the C ABI.
All computation happens in the library's HIP kernels; PyTorch provides device
memory and streams.
"""
from __future__ import annotations

import ctypes
from dataclasses import dataclass

import torch

from ._lib import (QD_EPI_NONE, QD_EPI_SILU, QD_FMT_FP16, QD_FMT_INT4_G64, QD_FMT_INT8_B32, QD_MAX_K,
                   QD_MAX_M, QD_PRO_GLU, QD_PRO_NONE, QD_PRO_RMSNORM, QDError, QDLinearOp, QDWeight,
                   check, lib)

__all__ = [
    "FORMATS", "PackedWeight", "QDError", "packed_bytes", "qpack_int8_b32", "qpack_int4_g64",
    "qpack_fp16", "qgemv_int8_b32", "qgemv_int4_g64", "qgemv_fp16", "qgemm_small_m", "decode_linear_stack", "StackPlan",
    "stack_run_noalloc",
    "QD_MAX_K", "QD_MAX_M", "LinearOp", "PROLOGUES", "EPILOGUES",
]

FORMATS = {"int8_b32": QD_FMT_INT8_B32, "int4_g64": QD_FMT_INT4_G64, "fp16": QD_FMT_FP16}
_PACK = {"int8_b32": "qpack_int8_b32", "int4_g64": "qpack_int4_g64", "fp16": "qpack_fp16"}
_GEMV = {"int8_b32": "qgemv_int8_b32", "int4_g64": "qgemv_int4_g64", "fp16": "qgemv_fp16"}


def _stream() -> int:
    return torch.cuda.current_stream().cuda_stream


def _ptr(t: torch.Tensor | None) -> int | None:
    return None if t is None else t.data_ptr()


def packed_bytes(fmt: str, n: int, k: int) -> int:
    """Size in bytes of the tiled blob for an [n, k] matrix (0 if invalid)."""
    return int(lib.qd_packed_bytes(FORMATS[fmt], n, k))


@dataclass
class PackedWeight:
    """A quantized matrix in the library's tiled layout (device uint8 blob)."""
    fmt: str
    n: int
    k: int
    blob: torch.Tensor

    def desc(self) -> QDWeight:
        return QDWeight(FORMATS[self.fmt], 0, self.n, self.k, _ptr(self.blob), self.blob.numel())


def _check_cuda(t: torch.Tensor, dtype, name: str) -> None:
    if not isinstance(t, torch.Tensor) or t.device.type != "cuda":
        raise TypeError(f"{name} must be a CUDA/HIP tensor")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _pack(fmt: str, w: torch.Tensor, out: torch.Tensor | None, err: torch.Tensor | None,
          check_errors: bool) -> PackedWeight:
    _check_cuda(w, torch.float32, "w")
    if w.dim() != 2:
        raise ValueError("w must be [N, K]")
    n, k = w.shape
    size = packed_bytes(fmt, n, k)
    if out is None:
        out = torch.empty(size, dtype=torch.uint8, device=w.device)
    else:
        _check_cuda(out, torch.uint8, "out")
    own_flag = err is None
    if own_flag:
        err = torch.zeros(1, dtype=torch.int32, device=w.device)
    fn = getattr(lib, _PACK[fmt])
    check(fn(_ptr(w), n, k, _ptr(out), out.numel(), _ptr(err), _stream()), _PACK[fmt])
    if check_errors and own_flag:
        flag = int(err.item())
        if flag:
            raise QDError(4, f"{_PACK[fmt]} (device flag {flag})")
    return PackedWeight(fmt, n, k, out)


def qpack_int8_b32(w: torch.Tensor, out: torch.Tensor | None = None,
                   err: torch.Tensor | None = None, check_errors: bool = True) -> PackedWeight:
    """Quantize fp32 [N, K] (device) to int8 b32 and pack it (bit-exact)."""
    return _pack("int8_b32", w, out, err, check_errors)


def qpack_int4_g64(w: torch.Tensor, out: torch.Tensor | None = None,
                   err: torch.Tensor | None = None, check_errors: bool = True) -> PackedWeight:
    """Quantize fp32 [N, K] (device) to affine int4 g64 and pack it (bit-exact)."""
    return _pack("int4_g64", w, out, err, check_errors)


def qpack_fp16(w: torch.Tensor, out: torch.Tensor | None = None,
               err: torch.Tensor | None = None, check_errors: bool = True) -> PackedWeight:
    """Round fp32 [N, K] (device) to fp16 and pack it in the tiled layout (bit-exact)."""
    return _pack("fp16", w, out, err, check_errors)


def _gemv(fmt: str, w: PackedWeight, x: torch.Tensor, y: torch.Tensor | None) -> torch.Tensor:
    if w.fmt != fmt:
        raise ValueError(f"weight is {w.fmt}, entry point wants {fmt}")
    _check_cuda(x, torch.float16, "x")
    if x.numel() != w.k:
        raise ValueError("x must hold K values")
    if y is None:
        y = torch.empty(w.n, dtype=torch.float16, device=x.device)
    else:
        _check_cuda(y, torch.float16, "y")
        if y.numel() != w.n:
            raise ValueError("y must hold N values")
    d = w.desc()
    fn = getattr(lib, _GEMV[fmt])
    check(fn(ctypes.byref(d), _ptr(x), _ptr(y), _stream()), _GEMV[fmt])
    return y


def qgemv_int8_b32(w: PackedWeight, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = W^ x for one token; x fp16 [K] -> y fp16 [N]."""
    return _gemv("int8_b32", w, x, y)


def qgemv_int4_g64(w: PackedWeight, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = W^ x for one token; x fp16 [K] -> y fp16 [N]."""
    return _gemv("int4_g64", w, x, y)


def qgemv_fp16(w: PackedWeight, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """y = W x for one token with fp16 weights; x fp16 [K] -> y fp16 [N]."""
    return _gemv("fp16", w, x, y)


def qgemm_small_m(w: PackedWeight, x: torch.Tensor, y: torch.Tensor | None = None) -> torch.Tensor:
    """Y = X W^T for m <= 16 tokens; X fp16 [m, K] -> Y fp16 [m, N]."""
    _check_cuda(x, torch.float16, "x")
    if x.dim() != 2 or x.shape[1] != w.k:
        raise ValueError("x must be [m, K]")
    m = x.shape[0]
    if y is None:
        y = torch.empty((m, w.n), dtype=torch.float16, device=x.device)
    else:
        _check_cuda(y, torch.float16, "y")
        if tuple(y.shape) != (m, w.n):
            raise ValueError("y must be [m, N]")
    d = w.desc()
    check(lib.qgemm_small_m(ctypes.byref(d), _ptr(x), _ptr(y), m, _stream()), "qgemm_small_m")
    return y


PROLOGUES = {"none": QD_PRO_NONE, "rmsnorm": QD_PRO_RMSNORM, "glu": QD_PRO_GLU}
EPILOGUES = {"none": QD_EPI_NONE, "silu": QD_EPI_SILU}


@dataclass
class LinearOp:
    """One projection of a decode step: y = W^ x.  Ops with equal `group`
    (consecutive) share x and run fused.

    prologue "rmsnorm" multiplies fp16(gamma * fp16(x * r)), r = 1 /
    sqrt(mean(x^2) + eps) per token; "glu" takes x as two blocks of [m, K]
    (A then B) and multiplies fp16(A * B).  epilogue "silu" stores
    fp16(silu(fp16(W^ u))).  The formulas are in include/qdecode.h."""
    w: PackedWeight
    x: torch.Tensor
    y: torch.Tensor
    group: int
    prologue: str = "none"
    gamma: torch.Tensor | None = None
    eps: float = 0.0
    epilogue: str = "none"


def _op_array(ops):
    arr = (QDLinearOp * max(1, len(ops)))()
    for i, op in enumerate(ops):
        arr[i] = QDLinearOp(op.w.desc(), _ptr(op.x), _ptr(op.y), op.group, PROLOGUES[op.prologue],
                            _ptr(op.gamma) if op.gamma is not None else None, op.eps,
                            EPILOGUES[op.epilogue])
    return arr


def decode_linear_stack(ops, m: int = 1) -> None:
    """Run one decode step's projections back to back on the current stream."""
    arr = _op_array(ops)
    check(lib.decode_linear_stack(arr, len(ops), m, _stream()), "decode_linear_stack")


def describe_stack_plan(ops, m: int = 1, workgroups: int | None = None) -> list:
    """Diagnostics: the int64 words of qd_stack_plan_describe for `ops`, the
    schedule a plan gets on a device of `workgroups` compute units (default:
    the current device's).  Host-only; the word layout is in
    include/qdecode.h."""
    if workgroups is None:
        workgroups = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    arr = _op_array(ops)
    n = ctypes.c_int64(0)
    check(lib.qd_stack_plan_describe(arr, len(ops), m, workgroups, None, 0, ctypes.byref(n)),
          "qd_stack_plan_describe")
    buf = (ctypes.c_int64 * n.value)()
    check(lib.qd_stack_plan_describe(arr, len(ops), m, workgroups, buf, n.value, ctypes.byref(n)),
          "qd_stack_plan_describe")
    return list(buf)


class StackPlan:
    """A validated decode step kept on the device; run() enqueues one step.

    The tensors referenced by `ops` must outlive the plan."""

    def __init__(self, ops, m: int = 1):
        self._ops = list(ops)          # keep tensors alive
        arr = _op_array(self._ops)
        h = ctypes.c_void_p()
        check(lib.qd_stack_plan_create(arr, len(self._ops), m, ctypes.byref(h)), "qd_stack_plan_create")
        self._h = h

    def run(self) -> None:
        check(lib.qd_stack_plan_run(self._h, _stream()), "qd_stack_plan_run")

    def error(self) -> int:
        e = ctypes.c_int32(0)
        check(lib.qd_stack_plan_error(self._h, ctypes.byref(e)), "qd_stack_plan_error")
        return e.value

    @property
    def persistent(self) -> bool:
        """True if runs use the persistent kernel (one launch per step; at
        m > 1 a small activation-copy launch first), False if they replay the
        per-group launches."""
        v = ctypes.c_int32(0)
        check(lib.qd_stack_plan_is_persistent(self._h, ctypes.byref(v)), "qd_stack_plan_is_persistent")
        return bool(v.value)

    def set_spin_limit(self, polls: int) -> None:
        """Diagnostics: bound every wait of the persistent kernel by `polls`
        polls for the following runs (default 2**20, about a second)."""
        check(lib.qd_stack_plan_set_spin_limit(self._h, polls), "qd_stack_plan_set_spin_limit")

    def close(self) -> None:
        if getattr(self, "_h", None) is not None and self._h.value:
            lib.qd_stack_plan_destroy(self._h)
            self._h = ctypes.c_void_p()

    def __del__(self):
        try:
            self.close()
        except Exception:
            pass


def stack_run_noalloc(ops, m: int = 1, err: torch.Tensor | None = None) -> None:
    """One step of `ops` in the persistent kernel without a plan object and
    without allocating device memory (tables and scratch in the library's
    static per-device array).  `err`, an int32 CUDA tensor, gets the run's
    error bits OR-ed in.  Calls overlapping on one device race."""
    if err is not None and not (err.is_cuda and err.dtype == torch.int32 and err.numel() >= 1):
        raise ValueError("err must be an int32 CUDA tensor")
    arr = _op_array(ops)
    check(lib.qd_stack_run_noalloc(arr, len(ops), m, _ptr(err), _stream()), "qd_stack_run_noalloc")


def read_probe(buf: torch.Tensor, sink: torch.Tensor, grid: int = 512) -> None:
    """Enqueue one plain streaming read of every byte of `buf` (a measurement
    helper: the bandwidth a bare read reaches, to quote a step against).
    `sink` is a 4-byte int32 device tensor the kernel writes only if an
    impossible value turns up."""
    if not (buf.is_cuda and sink.is_cuda and sink.dtype == torch.int32 and sink.numel() >= 1):
        raise ValueError("read_probe needs a CUDA buffer and an int32 CUDA sink")
    nbytes = buf.numel() * buf.element_size()
    check(lib.qd_read_probe(buf.data_ptr(), nbytes, sink.data_ptr(), grid, _stream()), "qd_read_probe")
