"""Host-side checks of the C ABI (no GPU needed): the library loads, exports
every function include/qdecode.h declares, sizes blobs like the layout spec,
and rejects bad arguments before touching a device."""
import ctypes
import os
import re

import pytest

from oracle import layout

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.fixture(scope="module")
def L():
    from int4_quantized_decode_amd import _lib
    return _lib


def _declared_functions():
    text = open(os.path.join(ROOT, "include", "qdecode.h")).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    names = re.findall(r"\b([a-z_][a-z0-9_]*)\s*\([^;{]*\)\s*;", text)
    return sorted(set(names))


def test_exports_every_declared_function(L):
    names = _declared_functions()
    assert {"qgemv_int8_b32", "qgemv_int4_g64", "qgemm_small_m", "decode_linear_stack",
            "qpack_int8_b32", "qpack_int4_g64", "qd_packed_bytes"} <= set(names)
    for n in names:
        assert hasattr(L.lib, n), n
        assert n in L.SIGNATURES, n


@pytest.mark.parametrize("fmt,code", [("int8_b32", 1), ("int4_g64", 2), ("fp16", 3)])
@pytest.mark.parametrize("n,k", [(16, 256), (37, 576), (151936, 4096), (1, 64), (4096, 12288)])
def test_packed_bytes_matches_layout_spec(L, fmt, code, n, k):
    assert L.lib.qd_packed_bytes(code, n, k) == layout.packed_bytes(fmt, n, k)


def test_packed_bytes_rejects(L):
    assert L.lib.qd_packed_bytes(1, 16, 48) == 0          # K % 32
    assert L.lib.qd_packed_bytes(2, 16, 96) == 0          # K % 64
    assert L.lib.qd_packed_bytes(3, 16, 48) == 0          # fp16: K % 32
    assert L.lib.qd_packed_bytes(4, 16, 256) == 0         # unknown format
    assert L.lib.qd_packed_bytes(1, -1, 256) == 0
    assert L.lib.qd_packed_bytes(1, 16, L.QD_MAX_K + 256) == 0


def test_status_strings(L):
    for s in range(0, 9):
        assert L.lib.qd_status_string(s)


def _w(L, fmt=1, n=32, k=256, data=4096, nbytes=None):
    nb = L.lib.qd_packed_bytes(fmt, n, k) if nbytes is None else nbytes
    return L.QDWeight(fmt, 0, n, k, data, nb)


def test_gemv_validation_errors(L):
    lib = L.lib
    x, y = 1 << 20, 1 << 24
    assert lib.qgemv_int8_b32(None, x, y, None) == 1                            # EINVAL
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L, fmt=2)), x, y, None) == 6      # EFORMAT
    assert lib.qgemv_int4_g64(ctypes.byref(_w(L, fmt=1)), x, y, None) == 6
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L, k=48)), x, y, None) == 2       # ESHAPE
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L, nbytes=100)), x, y, None) == 2
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L, data=4100)), x, y, None) == 3  # EALIGN
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L)), x + 2, y, None) == 3
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L)), None, y, None) == 1
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L)), x, None, None) == 1
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L)), x, x, None) == 1             # y overlaps x
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L, data=0)), x, y, None) == 1
    assert lib.qgemv_int8_b32(ctypes.byref(_w(L, n=0)), None, None, None) == 0  # empty: no-op


def test_small_m_validation_errors(L):
    lib = L.lib
    x, y = 1 << 20, 1 << 24
    assert lib.qgemm_small_m(ctypes.byref(_w(L)), x, y, 0, None) == 2
    assert lib.qgemm_small_m(ctypes.byref(_w(L)), x, y, 17, None) == 2
    assert lib.qgemm_small_m(ctypes.byref(_w(L, fmt=2, k=96)), x, y, 4, None) == 2   # int4: K % 64


def test_pack_validation_errors(L):
    lib = L.lib
    w, out = 1 << 20, 1 << 26
    need = lib.qd_packed_bytes(1, 32, 256)
    assert lib.qpack_int8_b32(w, 32, 48, out, need, None, None) == 2
    assert lib.qpack_int8_b32(w, 32, 256, out, need - 1, None, None) == 2
    assert lib.qpack_int8_b32(w + 4, 32, 256, out, need, None, None) == 3
    assert lib.qpack_int8_b32(w, 32, 256, out + 8, need, None, None) == 3
    assert lib.qpack_int8_b32(None, 32, 256, out, need, None, None) == 1
    assert lib.qpack_int4_g64(w, 32, 96, out, need, None, None) == 2
    assert lib.qpack_int8_b32(w, 0, 256, None, 0, None, None) == 0            # empty


def test_stack_validation_errors(L):
    lib = L.lib
    ops = (L.QDLinearOp * 2)()
    ops[0] = L.QDLinearOp(_w(L), 1 << 20, 1 << 24, 0, 0)
    ops[1] = L.QDLinearOp(_w(L, k=512, nbytes=L.lib.qd_packed_bytes(1, 32, 512)), 1 << 20,
                          1 << 25, 0, 0)                                      # same group, other K
    assert lib.decode_linear_stack(ops, 2, 1, None) == 1
    assert lib.decode_linear_stack(ops, 1, 0, None) == 2                      # m out of range
    assert lib.decode_linear_stack(None, 1, 1, None) == 1
    ops[1] = L.QDLinearOp(_w(L, fmt=2, k=96), 1 << 20, 1 << 25, 1, 0)
    assert lib.decode_linear_stack(ops, 2, 4, None) == 2                      # int4 needs K % 64
    h = ctypes.c_void_p()
    assert lib.qd_stack_plan_create(ops, 2, 0, ctypes.byref(h)) == 2
    assert lib.qd_stack_plan_create(ops, 2, 1, None) == 1
    assert lib.qd_stack_plan_run(None, None) == 1
    v = ctypes.c_int32(5)
    assert lib.qd_stack_plan_is_persistent(None, ctypes.byref(v)) == 1
    assert lib.qd_stack_plan_set_spin_limit(None, 0) == 1


def test_read_probe_validation_errors(L):
    lib = L.lib
    buf, sink = 1 << 20, 1 << 24
    assert lib.qd_read_probe(None, 64, sink, 4, None) == 1                    # EINVAL
    assert lib.qd_read_probe(buf, 64, None, 4, None) == 1
    assert lib.qd_read_probe(buf + 8, 64, sink, 4, None) == 3                 # EALIGN
    assert lib.qd_read_probe(buf, 64, sink + 2, 4, None) == 3
    assert lib.qd_read_probe(buf, 0, sink, 4, None) == 2                      # ESHAPE
    assert lib.qd_read_probe(buf, 64, sink, 0, None) == 2
    assert lib.qd_read_probe(buf, 64, sink, 65536, None) == 2


def test_stack_glue_validation_errors(L):
    """Prologue and epilogue fields are checked before anything is enqueued."""
    lib = L.lib
    x, y, gam = 1 << 20, 1 << 24, 1 << 26

    def one(**kw):
        f = dict(w=_w(L), x=x, y=y, group=0, prologue=0, gamma=None, eps=0.0, epilogue=0)
        f.update(kw)
        arr = (L.QDLinearOp * 1)()
        arr[0] = L.QDLinearOp(f["w"], f["x"], f["y"], f["group"], f["prologue"], f["gamma"],
                              f["eps"], f["epilogue"])
        return lib.decode_linear_stack(arr, 1, 1, None)

    assert one(prologue=3) == 1                                   # unknown prologue
    assert one(epilogue=2) == 1                                   # unknown epilogue
    assert one(prologue=1, gamma=None, eps=1e-6) == 1             # RMSNorm without gamma
    assert one(prologue=1, gamma=gam, eps=0.0) == 1               # eps must be > 0
    assert one(prologue=1, gamma=gam, eps=float("nan")) == 1
    assert one(prologue=1, gamma=gam, eps=float("inf")) == 1
    assert one(prologue=1, gamma=gam + 8, eps=1e-6) == 3          # gamma alignment
    assert one(prologue=1, gamma=y, eps=1e-6) == 1                # gamma overlaps y
    assert one(prologue=0, gamma=gam) == 1                        # gamma without RMSNorm
    assert one(prologue=2, eps=1e-6) == 1                         # eps without RMSNorm
    # a gated product reads 2 x K halves: y just past K halves overlaps it
    assert one(prologue=2, y=x + 256 * 2) == 1
    assert one(prologue=0, w=_w(L, n=0), y=x + 256 * 2) == 0      # N == 0: nothing to run

    arr = (L.QDLinearOp * 2)()
    arr[0] = L.QDLinearOp(_w(L), x, y, 0, 1, gam, 1e-6, 0)
    arr[1] = L.QDLinearOp(_w(L), x, y + 4096, 0, 1, gam, 1e-5, 1)  # same group, other eps
    assert lib.decode_linear_stack(arr, 2, 1, None) == 1
    arr[1] = L.QDLinearOp(_w(L), x, y + 4096, 0, 0, None, 0.0, 1)  # same group, no prologue
    assert lib.decode_linear_stack(arr, 2, 1, None) == 1
    arr[1] = L.QDLinearOp(_w(L), y, x, 0, 1, gam, 1e-6, 0)         # other x; and y over op 0's x
    assert lib.decode_linear_stack(arr, 2, 1, None) == 1
    h = ctypes.c_void_p()
    assert lib.qd_stack_plan_create(arr, 2, 1, ctypes.byref(h)) == 1


def test_op_struct_layout(L):
    """The ctypes mirror of qd_linear_op has the C layout (80 bytes, eps and
    epilogue after the gamma pointer)."""
    assert ctypes.sizeof(L.QDLinearOp) == 80
    assert L.QDLinearOp.gamma.offset == 64 and L.QDLinearOp.eps.offset == 72
    assert L.QDLinearOp.epilogue.offset == 76
