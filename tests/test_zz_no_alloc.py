"""The step entry point that allocates nothing (qd_stack_run_noalloc) against
the plan it stands in for (qd_stack_plan_create + qd_stack_plan_run), and
both against the oracle: outputs bit-identical to the plan's, two calls in a
row with the second one smaller (the static array keeps the previous call's
contents), one and several token rows, a replayed fp16 tail, glue, the error
word and the size limit."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import linear, quant
from tests.numerics import check_vector

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"


@pytest.fixture(scope="module")
def qd():
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import int4_quantized_decode_amd as qd
    return qd


def _gpu(a):
    return torch.from_numpy(np.ascontiguousarray(a)).to(DEV)


def _host(t):
    torch.cuda.synchronize()
    return t.cpu().numpy()


PACK = {"int8_b32": quant.quantize_int8_b32, "int4_g64": quant.quantize_int4_g64, "fp16": quant.quantize_fp16}


def _decoder_ops(qd, fmt, m, layers, hidden, mlp, vocab, tag, head_fmt=None):
    d = si.Decoder(f"noalloc-{tag}", layers=layers, hidden=hidden, q_heads=hidden // 64, mlp=mlp, vocab=vocab,
                   kv_heads=2, head_dim=64)
    ops, meta = [], []
    for gid, (gname, members) in enumerate(d.groups()):
        k = members[0][2]
        x = si.activations(si.seed_for("noalloc-x", tag, gname, m), m, k)
        x_gpu = _gpu(x if m > 1 else x[0])
        for pname, n, kk in members:
            f = head_fmt if (pname == "head" and head_fmt) else fmt
            w = si.weights(si.seed_for("noalloc-w", tag, pname), n, kk)
            pw = {"int8_b32": qd.qpack_int8_b32, "int4_g64": qd.qpack_int4_g64, "fp16": qd.qpack_fp16}[f](_gpu(w))
            y = torch.full((m, n) if m > 1 else (n,), float("nan"), dtype=torch.float16, device=DEV)
            ops.append(qd.LinearOp(pw, x_gpu, y, gid))
            meta.append((pname, f, w, x))
    return ops, meta


def _run_both(qd, ops, m):
    """Plan outputs, then no-alloc outputs (outputs poisoned before each)."""
    plan = qd.StackPlan(ops, m)
    for op in ops:
        op.y.fill_(float("nan"))
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    want = [_host(op.y).copy() for op in ops]
    persistent = plan.persistent
    plan.close()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for op in ops:
        op.y.fill_(float("nan"))
    qd.stack_run_noalloc(ops, m, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    got = [_host(op.y).copy() for op in ops]
    return want, got, persistent


def _check(ops, meta, m, want, got):
    for a, b, (pname, f, w, x) in zip(want, got, meta):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16)), f"{pname}: differs from the plan"
        parts = PACK[f](w)
        y_ref = linear.ref_linear(f, parts, x)
        rmax = linear.row_max_abs(f, parts)
        for i in range(m):
            check_vector(b.reshape(m, -1)[i], y_ref[i], rmax, x[i], f"{pname} row {i}")


@pytest.mark.parametrize("fmt,m", [("int8_b32", 1), ("int4_g64", 1), ("int8_b32", 16), ("int4_g64", 16),
                                   ("int8_b32", 5)])
def test_noalloc_matches_plan_two_calls(qd, fmt, m):
    # first call: a larger step; second: a smaller one, over the same static array
    big, big_meta = _decoder_ops(qd, fmt, m, layers=3, hidden=512, mlp=1280, vocab=1000, tag="big")
    want, got, persistent = _run_both(qd, big, m)
    assert persistent
    _check(big, big_meta, m, want, got)
    small, small_meta = _decoder_ops(qd, fmt, m, layers=1, hidden=256, mlp=512, vocab=300, tag="small")
    want, got, persistent = _run_both(qd, small, m)
    assert persistent
    _check(small, small_meta, m, want, got)


@pytest.mark.parametrize("m", [1, 4])
def test_noalloc_persistent_prefix_and_fp16_tail(qd, m):
    ops, meta = _decoder_ops(qd, "int8_b32", m, layers=2, hidden=256, mlp=768, vocab=700, tag="tail",
                             head_fmt="fp16")
    want, got, persistent = _run_both(qd, ops, m)
    assert persistent
    _check(ops, meta, m, want, got)


def test_noalloc_glued_step(qd):
    """RMSNorm before q|k|v and gate|up, silu on gate, the gated product
    before down, chained through the layers: bit-identical to the plan (whose
    glue the glue tests check against the oracle)."""
    H, Q, KV, I = 256, 256, 128, 512
    eps = 1e-6
    ops, gid = [], 0
    x_in = _gpu(si.activations(si.seed_for("na-glue-x"), 1, H)[0])
    for layer in range(2):
        gam = _gpu(si.norm_weight(si.seed_for("na-gamma", layer), H))
        for name, n in (("q", Q), ("k", KV), ("v", KV)):
            w = si.weights(si.seed_for("na-glue", layer, name), n, H)
            ops.append(qd.LinearOp(qd.qpack_int8_b32(_gpu(w)), x_in, torch.empty(n, dtype=torch.float16, device=DEV),
                                   gid, prologue="rmsnorm", gamma=gam, eps=eps))
        gid += 1
        gu = torch.empty(2 * I, dtype=torch.float16, device=DEV)
        o_y = ops[-3].y
        w = si.weights(si.seed_for("na-glue", layer, "gate"), I, Q)
        ops.append(qd.LinearOp(qd.qpack_int8_b32(_gpu(w)), o_y, gu[:I], gid, prologue="rmsnorm", gamma=gam,
                               eps=eps, epilogue="silu"))
        w = si.weights(si.seed_for("na-glue", layer, "up"), I, Q)
        ops.append(qd.LinearOp(qd.qpack_int8_b32(_gpu(w)), o_y, gu[I:], gid, prologue="rmsnorm", gamma=gam,
                               eps=eps))
        gid += 1
        x_in = torch.empty(H, dtype=torch.float16, device=DEV)
        w = si.weights(si.seed_for("na-glue", layer, "down"), H, I)
        ops.append(qd.LinearOp(qd.qpack_int8_b32(_gpu(w)), gu, x_in, gid, prologue="glu"))
        gid += 1
    want, got, persistent = _run_both(qd, ops, 1)
    assert persistent
    for a, b in zip(want, got):
        assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    assert np.all(np.isfinite(got[-1].astype(np.float64)))


def test_noalloc_size_limit(qd):
    """More group records than the static array holds: a clear error, and
    nothing runs (the output keeps its poison)."""
    w = si.weights(si.seed_for("na-limit"), 16, 256)
    pw = qd.qpack_int8_b32(_gpu(w))
    x = _gpu(si.activations(si.seed_for("na-limit-x"), 1, 256)[0])
    y = torch.full((16,), float("nan"), dtype=torch.float16, device=DEV)
    ops = [qd.LinearOp(pw, x, y, g) for g in range(600)]
    with pytest.raises(qd.QDError) as e:
        qd.stack_run_noalloc(ops, 1)
    assert e.value.status == 2          # QD_ESHAPE
    assert np.all(np.isnan(_host(y).astype(np.float64)))
    # within the limit the same kind of step runs and matches the oracle
    qd.stack_run_noalloc(ops[:500], 1)
    parts = quant.quantize_int8_b32(w)
    xh = si.activations(si.seed_for("na-limit-x"), 1, 256)[0]
    check_vector(_host(y), linear.ref_linear("int8_b32", parts, xh), linear.row_max_abs("int8_b32", parts), xh,
                 "within limit")
