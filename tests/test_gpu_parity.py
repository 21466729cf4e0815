"""GPU parity: the HIP path against the CPU oracle on the same seeded inputs.

Packing is compared byte for byte; products within the acceptance bound of
tests/numerics.py.  Sizes span several tiles plus ragged row and K tails; the
full 8B-shaped matrices are checked on sampled rows."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import layout, linear, quant
from tests import hard_weights
from tests import test_oracle_pins as pins
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


FMTS = ["int8_b32", "int4_g64", "fp16"]


def _oracle_parts(fmt, w):
    return {"int8_b32": quant.quantize_int8_b32, "int4_g64": quant.quantize_int4_g64,
            "fp16": quant.quantize_fp16}[fmt](w)


def _oracle_blob(fmt, parts):
    return {"int8_b32": layout.tile_int8_b32, "int4_g64": layout.tile_int4_g64,
            "fp16": layout.tile_fp16}[fmt](*parts)


def _pack_fn(qd, fmt):
    return {"int8_b32": qd.qpack_int8_b32, "int4_g64": qd.qpack_int4_g64, "fp16": qd.qpack_fp16}[fmt]


def _pack(qd, fmt, w_gpu):
    return _pack_fn(qd, fmt)(w_gpu)


def _gemv_fn(qd, fmt):
    return {"int8_b32": qd.qgemv_int8_b32, "int4_g64": qd.qgemv_int4_g64, "fp16": qd.qgemv_fp16}[fmt]


SHAPES = [(16, 256), (200, 1056), (200, 1088), (37, 576), (1, 64), (48, 2048), (2048, 2048),
          (100, 4096)]


def _skip_bad_k(fmt, k):
    if fmt == "int4_g64" and k % 64:
        pytest.skip("int4 g64 needs K % 64 == 0")
    if k % 32:
        pytest.skip("K % 32 == 0 is required")


# ------------------------------------------------------------------ packing

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", SHAPES)
def test_pack_bit_exact(qd, fmt, n, k):
    _skip_bad_k(fmt, k)
    w = si.weights(si.seed_for("pack", fmt, n, k), n, k)
    pw = _pack(qd, fmt, _gpu(w))
    got = _host(pw.blob)
    want = _oracle_blob(fmt, _oracle_parts(fmt, w))
    assert got.size == want.size
    diff = np.flatnonzero(got != want)
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8]}"


def _adversarial(fmt, n=32, k=512, near_max=True):
    rng = np.random.default_rng(7)
    w = (rng.standard_normal((n, k)) * 0.02).astype(np.float32)
    w[0, :64] = 0.0                                          # zero blocks / groups
    s = np.float32(2.0 ** -7)
    w[1, :32] = (np.arange(32, dtype=np.float32) - 15.5) * s  # halves: exact ties
    w[1, 0] = np.float32(127) * s
    w[2, :] = (rng.standard_normal(k) * 1e-7).astype(np.float32)   # fp16-subnormal scales
    w[3, :] = (rng.standard_normal(k) * 50).astype(np.float32)     # large values
    w[4, :] = np.float32(0.3)                                       # constant groups
    w[5, 64:128] = -np.abs(w[5, 64:128])                           # one-signed groups
    w[6, :] = (rng.integers(-127, 128, k) * 2.0 ** -9).astype(np.float32)  # on-grid values
    for c in range(16):                                             # near-ties around x.5
        w[7, c] = np.float32((c + 0.5) * 2.0 ** -7 * (1 + (-1) ** c * 2.0 ** -20))
    w[7, 31] = np.float32(127 * 2.0 ** -7)
    # rows that reach the quantizers' clamps (subnormal int8 scales; INT4
    # groups whose fp16 min lands far from the true min) and signed zeros
    w[10:16, :] = hard_weights.int8_clamp_rows(k)
    w[16:22, :] = hard_weights.int4_clamp_rows(k)
    w[22:30, :] = hard_weights.signed_zero_rows(k)
    if fmt == "fp16":
        # exact midpoints between fp16 neighbours (ties), both signs, many exponents
        base = (rng.standard_normal(k) * np.exp2(rng.integers(-20, 12, k))).astype(np.float16)
        up = np.nextafter(base, np.float16(np.inf))
        w[8, :] = ((base.astype(np.float64) + up.astype(np.float64)) / 2).astype(np.float32)
        if near_max:                   # packing only: products would overflow fp16 outputs
            w[9, :] = np.float32(65504.0) * np.sign(rng.standard_normal(k)).astype(np.float32)
    return w


@pytest.mark.parametrize("fmt", FMTS)
def test_pack_adversarial_bit_exact(qd, fmt):
    w = _adversarial(fmt)
    # the oracle takes the clamp branches on these rows (both ends, both formats)
    if fmt == "int8_b32":
        hi, lo = pins._int8_clamp_events(w[10:16])
        assert hi > 0 and lo > 0
    if fmt == "int4_g64":
        hi, lo = pins._int4_clamp_events(w[16:22])
        assert hi > 0 and lo > 0
        assert (_oracle_parts(fmt, w)[2][22:30].view(np.uint16) == 0x8000).any()
    pw = _pack(qd, fmt, _gpu(w))
    got = _host(pw.blob)
    want = _oracle_blob(fmt, _oracle_parts(fmt, w))
    diff = np.flatnonzero(got != want)
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8]}"


@pytest.mark.parametrize("fmt", FMTS)
def test_pack_error_flags(qd, fmt):
    w = np.zeros((16, 256), np.float32)
    w[3, 7] = np.nan
    with pytest.raises(qd.QDError):
        _pack(qd, fmt, _gpu(w))
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    pack = _pack_fn(qd, fmt)
    pack(_gpu(w), err=err)
    assert int(err.item()) & 1
    # int8: max|w| / 127 beyond fp16; int4: the group min beyond fp16; fp16: the value
    w[3, 7] = {"int8_b32": 1e9, "int4_g64": -70000.0, "fp16": 65520.0}[fmt]
    err.zero_()
    pack(_gpu(w), err=err)
    assert int(err.item()) & 2


@pytest.mark.parametrize("fmt", FMTS)
def test_pack_without_error_flag(qd, fmt):
    """The error flag may be NULL: bad input is then only written as zeros."""
    import ctypes
    from int4_quantized_decode_amd import _lib
    w = si.weights(si.seed_for("noflag", fmt), 32, 256)
    w[5, 9] = np.nan
    wg = _gpu(w)
    n, k = w.shape
    out = torch.full((layout.packed_bytes(fmt, n, k),), 0xAB, dtype=torch.uint8, device=DEV)
    fn = getattr(_lib.lib, {"int8_b32": "qpack_int8_b32", "int4_g64": "qpack_int4_g64",
                            "fp16": "qpack_fp16"}[fmt])
    st = fn(wg.data_ptr(), n, k, out.data_ptr(), out.numel(), None,
            torch.cuda.current_stream().cuda_stream)
    assert st == 0
    got = _host(out)
    # the packer writes the block (int8: 32 values), group (int4: 64) or
    # 8-value run (fp16) holding the NaN as zeros, everything else as usual
    span = {"int8_b32": 32, "int4_g64": 64, "fp16": 8}[fmt]
    clean = w.copy()
    clean[5, 9 // span * span:(9 // span + 1) * span] = 0.0
    want = _oracle_blob(fmt, _oracle_parts(fmt, clean))
    diff = np.flatnonzero(got != want)
    assert diff.size == 0, f"{diff.size} bytes differ, first at {diff[:8]}"


# ------------------------------------------------------------------ M = 1

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n,k", SHAPES + [(16, 24576)])
def test_gemv_parity(qd, fmt, n, k):
    _skip_bad_k(fmt, k)
    w = si.weights(si.seed_for("gemv", fmt, n, k), n, k)
    x = si.activations(si.seed_for("gemv-x", fmt, n, k), 1, k)[0]
    pw = _pack(qd, fmt, _gpu(w))
    fn = _gemv_fn(qd, fmt)
    y = _host(fn(pw, _gpu(x)))
    parts = _oracle_parts(fmt, w)
    y_ref = linear.ref_linear(fmt, parts, x)
    check_vector(y, y_ref, linear.row_max_abs(fmt, parts), x, f"{fmt} {n}x{k}")


@pytest.mark.parametrize("fmt", FMTS)
def test_gemv_edge_cases(qd, fmt):
    fn = _gemv_fn(qd, fmt)
    # K = 0: y = 0
    pw0 = _pack(qd, fmt, torch.zeros((20, 0), dtype=torch.float32, device=DEV))
    y0 = fn(pw0, torch.zeros(0, dtype=torch.float16, device=DEV),
            torch.full((20,), 7.0, dtype=torch.float16, device=DEV))
    assert not _host(y0).any()
    # N = 0: no-op
    pwn = _pack(qd, fmt, torch.zeros((0, 256), dtype=torch.float32, device=DEV))
    assert fn(pwn, torch.zeros(256, dtype=torch.float16, device=DEV)).numel() == 0
    # all-zero weights give exact zeros; adversarial rows stay in bound
    w = _adversarial(fmt, near_max=False)
    x = si.activations(99, 1, w.shape[1])[0]
    y = _host(fn(_pack(qd, fmt, _gpu(w)), _gpu(x)))
    parts = _oracle_parts(fmt, w)
    check_vector(y, linear.ref_linear(fmt, parts, x), linear.row_max_abs(fmt, parts), x, "adv")


# ------------------------------------------------------------------ M <= 16

@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("m", [1, 5, 16])
@pytest.mark.parametrize("n,k", [(16, 256), (200, 1056), (48, 2048), (100, 4096), (64, 12288),
                                 (40, 1088), (24, 24576)])
def test_small_m_parity(qd, fmt, m, n, k):
    _skip_bad_k(fmt, k)
    w = si.weights(si.seed_for("sm", n, k), n, k)
    X = si.activations(si.seed_for("sm-x", m, n, k), m, k)
    pw = _pack(qd, fmt, _gpu(w))
    Y = _host(qd.qgemm_small_m(pw, _gpu(X)))
    parts = _oracle_parts(fmt, w)
    Y_ref = linear.ref_linear(fmt, parts, X)
    rmax = linear.row_max_abs(fmt, parts)
    for i in range(m):
        check_vector(Y[i], Y_ref[i], rmax, X[i], f"{fmt} m={m} row {i}")


@pytest.mark.parametrize("fmt", FMTS)
def test_small_m_rows_match_gemv(qd, fmt):
    """Each token row of the 16-row chunk agrees with the one-token GEMV on
    that row (the pages' chunked-vs-S=1 consistency idea)."""
    n, k = 512, 4096
    w = si.weights(5, n, k)
    X = si.activations(6, 16, k)
    pw = _pack(qd, fmt, _gpu(w))
    Y = _host(qd.qgemm_small_m(pw, _gpu(X)))
    parts = _oracle_parts(fmt, w)
    rmax = linear.row_max_abs(fmt, parts)
    gemv = _gemv_fn(qd, fmt)
    for i in range(16):
        y1 = _host(gemv(pw, _gpu(X[i])))
        check_vector(Y[i], y1.astype(np.float64), 2 * rmax, X[i], f"row {i}")


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("n_each", [8200, 32776])
def test_small_m_many_row_groups(qd, fmt, n_each):
    """At least 1024 row-groups: each workgroup takes two (below 2048 in the
    launch) or four row-groups that share one read of each activation block.
    Ragged last row-group, a fused pair whose workgroups straddle the member
    boundary (513 + 513 and 2049 + 2049 row-groups), and m below 16 (rows past
    m read as zero)."""
    from int4_quantized_decode_amd import LinearOp
    k = 2048
    n1, n2 = n_each, n_each                  # odd row-group counts, each ragged
    w1 = si.weights(si.seed_for("sm-many", 1), n1, k)
    w2 = si.weights(si.seed_for("sm-many", 2), n2, k)
    for m in (16, 5):
        X = si.activations(si.seed_for("sm-many-x", m), m, k)
        xg = _gpu(X)
        y1 = torch.full((m, n1), float("nan"), dtype=torch.float16, device=DEV)
        y2 = torch.full((m, n2), float("nan"), dtype=torch.float16, device=DEV)
        ops = [LinearOp(_pack(qd, fmt, _gpu(w1)), xg, y1, 0),
               LinearOp(_pack(qd, fmt, _gpu(w2)), xg, y2, 0)]
        qd.decode_linear_stack(ops, m)
        for w, y, name in ((w1, y1, "first"), (w2, y2, "second")):
            parts = _oracle_parts(fmt, w)
            Y_ref = linear.ref_linear(fmt, parts, X)
            rmax = linear.row_max_abs(fmt, parts)
            Yh = _host(y)
            for i in range(m):
                check_vector(Yh[i], Y_ref[i], rmax, X[i], f"{name} member m={m} row {i}")


# ------------------------------------------------------------------ stack

def _tiny_decoder_ops(qd, fmt, m, layers=2, chained=False):
    d = si.Decoder("tiny", layers=layers, hidden=512, q_heads=4, mlp=1280, vocab=1000,
                   kv_heads=2, head_dim=64)
    ops, meta = [], []
    gid = 0
    for gname, members in d.groups():
        k = members[0][2]
        x = si.activations(si.seed_for("stack-x", gname, m), m, k)
        x_gpu = _gpu(x if m > 1 else x[0])
        for pname, n, kk in members:
            w = si.weights(si.seed_for("stack-w", pname), n, kk)
            pw = _pack(qd, fmt, _gpu(w))
            y = torch.full((m, n) if m > 1 else (n,), float("nan"), dtype=torch.float16, device=DEV)
            ops.append(qd.LinearOp(pw, x_gpu, y, gid))
            meta.append((pname, w, x))
        gid += 1
    return ops, meta


@pytest.mark.parametrize("fmt,m", [("int8_b32", 1), ("int4_g64", 1), ("fp16", 1), ("int8_b32", 16),
                                   ("int4_g64", 16), ("fp16", 16)])
def test_stack_parity(qd, fmt, m):
    ops, meta = _tiny_decoder_ops(qd, fmt, m)
    qd.decode_linear_stack(ops, m)
    for op, (pname, w, x) in zip(ops, meta):
        y = _host(op.y)
        parts = _oracle_parts(fmt, w)
        y_ref = linear.ref_linear(fmt, parts, x)
        rmax = linear.row_max_abs(fmt, parts)
        if m == 1:
            check_vector(y, y_ref[0] if y_ref.ndim == 2 else y_ref, rmax, x[0], pname)
        else:
            for i in range(m):
                check_vector(y[i], y_ref[i], rmax, x[i], f"{pname} row {i}")


@pytest.mark.parametrize("m", [1, 16])
def test_stack_mixed_formats_fp16_head(qd, m):
    """The int8lin variant's step shape: int8 b32 body groups and an fp16 head
    group in one stack (per-group launches; the plan runs the body in the
    persistent kernel and replays the head's launch after it)."""
    ops, meta = _tiny_decoder_ops(qd, "int8_b32", m, layers=2)
    hidden = meta[-1][1].shape[1]
    w_head = si.weights(si.seed_for("fp16-head"), 1000, hidden)
    x_head = si.activations(si.seed_for("fp16-head-x", m), m, hidden)
    y_head = torch.full((m, 1000) if m > 1 else (1000,), float("nan"), dtype=torch.float16, device=DEV)
    head_op = qd.LinearOp(qd.qpack_fp16(_gpu(w_head)), _gpu(x_head if m > 1 else x_head[0]), y_head,
                          ops[-1].group + 1)
    ops = ops[:-1] + [head_op]                       # replace the int8 head
    meta = meta[:-1] + [("head16", w_head, x_head)]
    for use_plan in (False, True):
        for op in ops:
            op.y.fill_(float("nan"))
        if use_plan:
            plan = qd.StackPlan(ops, m)
            assert plan.persistent
            plan.run()
        else:
            qd.decode_linear_stack(ops, m)
        for op, (pname, w, x) in zip(ops, meta):
            fmt = "fp16" if pname == "head16" else "int8_b32"
            parts = _oracle_parts(fmt, w)
            Y = _host(op.y).reshape(m, -1)
            Y_ref = linear.ref_linear(fmt, parts, x).reshape(m, -1)
            rmax = linear.row_max_abs(fmt, parts)
            for t in range(m):
                check_vector(Y[t], Y_ref[t], rmax, x[t], f"{pname} token {t} plan={use_plan}")
        if use_plan:
            plan.close()


def _check_chain_on_device_inputs(bufs, parts_list, what):
    """Op i read bufs[i] and wrote bufs[i + 1]: each output against the
    oracle on the fp16 input the device actually read, at the acceptance
    bound.  (Read too early, an input would still hold its NaN poison.)"""
    vals = [_host(b).copy() for b in bufs]
    for i, parts in enumerate(parts_list):
        x_in = vals[i]
        assert np.all(np.isfinite(x_in.astype(np.float64))), f"{what}: input of op {i}"
        y_ref = linear.ref_linear("int8_b32", parts, x_in)
        check_vector(vals[i + 1], y_ref, linear.row_max_abs("int8_b32", parts), x_in, f"{what} op {i}")


def test_stack_chain_respects_order(qd):
    """A chain where each op reads the previous op's output: correct only if
    every group starts after the one before it has finished.  Outputs are
    poisoned with NaN first, so reading too early cannot pass."""
    from int4_quantized_decode_amd import LinearOp
    k = 1024
    ws = [si.weights(si.seed_for("chain", i), k, k) for i in range(4)]
    x0 = si.activations(si.seed_for("chain-x"), 1, k)[0]
    pws = [qd.qpack_int8_b32(_gpu(w)) for w in ws]
    bufs = [_gpu(x0)] + [torch.full((k,), float("nan"), dtype=torch.float16, device=DEV)
                         for _ in ws]
    ops = [LinearOp(pws[i], bufs[i], bufs[i + 1], i) for i in range(len(ws))]
    for rep in range(3):
        for b in bufs[1:]:
            b.fill_(float("nan"))
        qd.decode_linear_stack(ops, 1)
        _check_chain_on_device_inputs(bufs, [quant.quantize_int8_b32(w) for w in ws], f"chain rep {rep}")


# ------------------------------------------------------------------ full size, sampled

FULL = [("q", 4096, 4096), ("down", 4096, 12288), ("head", 151936, 4096)]


@pytest.mark.parametrize("fmt", FMTS)
@pytest.mark.parametrize("name,n,k", FULL)
def test_full_size_sampled(qd, fmt, name, n, k):
    """8B-shaped matrices at full size, in the launch configuration the bench
    uses; packing and outputs checked on sampled row-groups."""
    seed = si.matrix_seed("qwen3-8b", f"L0.{name}" if name != "head" else "head")
    w_gpu = si.weights_torch(seed, n, k, DEV)
    pw = _pack(qd, fmt, w_gpu)
    x = si.activations(si.seed_for("full-x", name), 1, k)[0]
    fn = _gemv_fn(qd, fmt)
    y = _host(fn(pw, _gpu(x)))
    rng = np.random.default_rng(3)
    R = -(-n // 16)
    rgs = sorted(set([0, R - 1] + list(rng.choice(R, 6, replace=False))))
    for r in rgs:
        rows = np.arange(16 * r, min(n, 16 * r + 16))
        w_rows = w_gpu[rows[0]:rows[-1] + 1].cpu().numpy()
        parts = _oracle_parts(fmt, w_rows)
        want = _oracle_blob(fmt, parts)
        got = _host(pw.blob[layout.row_group_slice(fmt, n, k, r)])
        assert np.array_equal(got, want), f"row-group {r} bytes differ"
        y_ref = linear.ref_linear(fmt, parts, x)
        check_vector(y[rows], y_ref, linear.row_max_abs(fmt, parts), x, f"{name} rg {r}")
    del w_gpu
    torch.cuda.empty_cache()


# ------------------------------------------------------------------ persistent plan

@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
def test_plan_parity_and_determinism(qd, fmt):
    """The persistent one-launch step: oracle parity on every output, repeated
    runs (outputs poisoned in between) are bit-identical, no wait timed out."""
    ops, meta = _tiny_decoder_ops(qd, fmt, 1, layers=3)
    plan = qd.StackPlan(ops, 1)
    assert plan.persistent
    first = None
    for rep in range(3):
        for op in ops:
            op.y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        outs = [_host(op.y).copy() for op in ops]
        if first is None:
            first = outs
            for y, (pname, w, x) in zip(outs, meta):
                parts = _oracle_parts(fmt, w)
                y_ref = linear.ref_linear(fmt, parts, x)[0]
                check_vector(y, y_ref, linear.row_max_abs(fmt, parts), x[0], f"plan {pname}")
        else:
            for a, b in zip(first, outs):
                assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    plan.close()


def test_plan_chain_respects_order(qd):
    """Each op reads the previous op's output inside one persistent launch."""
    from int4_quantized_decode_amd import LinearOp
    k = 1024
    depth = 6
    ws = [si.weights(si.seed_for("pchain", i), k, k) for i in range(depth)]
    x0 = si.activations(si.seed_for("pchain-x"), 1, k)[0]
    pws = [qd.qpack_int8_b32(_gpu(w)) for w in ws]
    bufs = [_gpu(x0)] + [torch.full((k,), float("nan"), dtype=torch.float16, device=DEV)
                         for _ in ws]
    ops = [LinearOp(pws[i], bufs[i], bufs[i + 1], i) for i in range(depth)]
    plan = qd.StackPlan(ops, 1)
    oracle_ops = [{"fmt": "int8_b32", "parts": quant.quantize_int8_b32(ws[0]), "x": x0}]
    oracle_ops += [{"fmt": "int8_b32", "parts": quant.quantize_int8_b32(ws[i]), "x_from": i - 1}
                   for i in range(1, depth)]
    for rep in range(3):
        for b in bufs[1:]:
            b.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        _check_chain_on_device_inputs(bufs, [op_["parts"] for op_ in oracle_ops], f"plan chain rep {rep}")
        # and the chain as a whole follows the oracle's own chain
        assert np.all(np.isfinite(_host(bufs[-1]).astype(np.float64)))
    plan.close()


def test_plan_ragged_and_uneven_groups(qd):
    """Groups with fewer row-groups than workgroups (most workgroups get none),
    long K up to the largest accepted (activations staged in many 1 KiB blocks), K that is not a multiple
    of 256 or gives an odd number of 256-wide blocks, ragged row tails, and
    groups with more row-groups than workgroups whose ranges straddle member
    boundaries."""
    from int4_quantized_decode_amd import LinearOp
    shapes = [[(24, 12288)], [(37, 2048), (5, 2048), (100, 2048)], [(4000, 512)], [(16, 256)],
              [(9, 4096)], [(40, 768)], [(33, 1056)], [(20, 24576)],      # the largest K
              # at least one row-group per workgroup: whole-row-group ranges, several of
              # which straddle a boundary between members
              [(4096, 256), (1024, 256), (1024, 256)], [(2000, 512), (1000, 512), (1200, 512)]]
    ops, meta = [], []
    for gi, members in enumerate(shapes):
        k = members[0][1]
        x = si.activations(si.seed_for("ragged-x", gi), 1, k)[0]
        xg = _gpu(x)
        for mi, (n, kk) in enumerate(members):
            w = si.weights(si.seed_for("ragged-w", gi, mi), n, kk)
            y = torch.full((n,), float("nan"), dtype=torch.float16, device=DEV)
            ops.append(LinearOp(qd.qpack_int8_b32(_gpu(w)), xg, y, gi))
            meta.append((w, x))
    plan = qd.StackPlan(ops, 1)
    assert plan.persistent
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    for op, (w, x) in zip(ops, meta):
        parts = quant.quantize_int8_b32(w)
        check_vector(_host(op.y), linear.ref_linear("int8_b32", parts, x),
                     linear.row_max_abs("int8_b32", parts), x, f"ragged {w.shape}")
    plan.close()


def test_plan_replays_launches_when_schedule_exceeds_lds(qd):
    """A step with more groups than one CU's LDS can hold the schedule of is
    replayed as per-group launches: same results, reported as not persistent."""
    from int4_quantized_decode_amd import LinearOp
    n_groups, n, k = 2600, 16, 256
    w_all = si.weights(si.seed_for("many-groups-w"), n_groups * n, k)
    x_all = si.activations(si.seed_for("many-groups-x"), n_groups, k)
    pw_all = [qd.qpack_int8_b32(_gpu(w_all[i * n:(i + 1) * n])) for i in range(n_groups)]
    xg = _gpu(x_all)
    y = torch.full((n_groups, n), float("nan"), dtype=torch.float16, device=DEV)
    ops = [LinearOp(pw_all[i], xg[i], y[i], i) for i in range(n_groups)]
    plan = qd.StackPlan(ops, 1)
    assert not plan.persistent
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    yh = _host(y)
    for i in range(0, n_groups, 97):
        parts = quant.quantize_int8_b32(w_all[i * n:(i + 1) * n])
        check_vector(yh[i], linear.ref_linear("int8_b32", parts, x_all[i]),
                     linear.row_max_abs("int8_b32", parts), x_all[i], f"replayed group {i}")
    plan.close()


def _sample_picks(decoder):
    last, mid = decoder.layers - 1, decoder.layers // 2
    return ["L0.q", "L0.k", f"L{mid}.gate", f"L{mid}.up", f"L{last}.down", f"L{last}.o", "head"]


def test_single_gemv_config_bench_path(qd):
    """The single 2048 x 2048 int8 GEMV configuration through the bench's own
    builder and launch path (qgemv via decode_linear_stack), every output
    against the oracle."""
    import bench
    ops, alg_bytes, weight_bytes, m = bench.build_stack(qd, si, torch, "gemv-2048x2048-int8", DEV)
    assert len(ops) == 1 and m == 1
    op = ops[0]
    op.y.fill_(float("nan"))
    qd.decode_linear_stack(ops, 1)
    torch.cuda.synchronize()
    w = si.weights_torch(si.matrix_seed("single", "W"), 2048, 2048, DEV).cpu().numpy()
    parts = quant.quantize_int8_b32(w)
    x = op.x.cpu().numpy()
    check_vector(_host(op.y), linear.ref_linear("int8_b32", parts, x), linear.row_max_abs("int8_b32", parts),
                 x, "C1 2048x2048")


@pytest.mark.parametrize("workload", ["qwen3-8b-int8-m1", "qwen3-8b-int4-m1", "qwen3.8-27b-int8-m1",
                                      "qwen3-2b-int8-m1", "qwen3-4b-int8-m1",
                                      "qwen3-8b-int8-chain-m1", "qwen3-8b-int8-m16",
                                      "qwen3-8b-int8-chain-m16",
                                      "qwen3-8b-int4-m16",
                                      "qwen3.8-27b-int8-m16"])
def test_plan_full_size_sampled(qd, workload):
    """The full decoder-shaped step in the launch configuration the bench
    times: every output finite, sampled rows of sampled projections match
    the oracle (every token row at m = 16)."""
    import bench
    ops, alg_bytes, weight_bytes, m = bench.build_stack(qd, si, torch, workload, DEV)
    plan = qd.StackPlan(ops, m)
    for op in ops:
        op.y.fill_(float("nan"))
    plan.run()
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    wl = si.WORKLOADS[workload]
    names = [p for _, ms in wl.decoder.groups() for p, _, _ in ms]
    for op in ops:
        assert torch.isfinite(op.y).all()
    assert plan.persistent
    picks = _sample_picks(wl.decoder)
    rng = np.random.default_rng(11)
    for name in picks:
        i = names.index(name)
        op = ops[i]
        n, k = op.w.n, op.w.k
        rows = np.sort(rng.choice(n, 24, replace=False))
        w_full = si.weights_torch(si.matrix_seed(wl.decoder.name, name), n, k, DEV)
        if wl.chain:                                   # the chained step's weight scale
            w_full.mul_(1.0 / (si.W_STD * k ** 0.5))
        w_rows = w_full[rows].cpu().numpy()
        del w_full
        x = op.x.cpu().numpy().reshape(m, k)           # the activations the op read
        parts = _oracle_parts(wl.fmt, w_rows)
        y_ref = linear.ref_linear(wl.fmt, parts, x).reshape(m, -1)
        y_got = _host(op.y).reshape(m, n)[:, rows]
        for t in range(m):
            check_vector(y_got[t], y_ref[t], linear.row_max_abs(wl.fmt, parts), x[t], f"{name} token {t}")
    plan.close()
    del ops
    torch.cuda.empty_cache()


@pytest.mark.parametrize("workload", ["qwen3-8b-int8-m16", "qwen3-8b-int4-m16", "qwen3.8-27b-int8-m16"])
def test_stack_full_size_sampled_m16(qd, workload):
    """The full 16-token chunked-prefill step as the bench times it (per-group
    MFMA launches): every output finite, sampled rows of sampled projections
    match the oracle for all 16 tokens."""
    import bench
    ops, alg_bytes, weight_bytes, m = bench.build_stack(qd, si, torch, workload, DEV)
    assert m == 16
    for op in ops:
        op.y.fill_(float("nan"))
    qd.decode_linear_stack(ops, m)
    torch.cuda.synchronize()
    wl = si.WORKLOADS[workload]
    names = [p for _, ms in wl.decoder.groups() for p, _, _ in ms]
    for op in ops:
        assert torch.isfinite(op.y).all()
    rng = np.random.default_rng(12)
    for name in _sample_picks(wl.decoder):
        op = ops[names.index(name)]
        n, k = op.w.n, op.w.k
        rows = np.sort(rng.choice(n, 16, replace=False))
        w_rows = si.weights_torch(si.matrix_seed(wl.decoder.name, name), n, k, DEV)[rows].cpu().numpy()
        X = op.x.cpu().numpy()
        parts = _oracle_parts(wl.fmt, w_rows)
        Y_ref = linear.ref_linear(wl.fmt, parts, X)
        Y = _host(op.y)[:, rows]
        rmax = linear.row_max_abs(wl.fmt, parts)
        for t in range(16):
            check_vector(Y[t], Y_ref[t], rmax, X[t], f"{name} token {t}")


def test_stack_full_size_sampled_fp16_head(qd):
    """The full 2B-shaped int8lin step (int8 b32 body, fp16 head 151936 x 2048)
    as the bench times it: outputs finite, sampled rows match the oracle."""
    import bench
    workload = "qwen3-2b-int8-fp16head-m1"
    ops, alg_bytes, weight_bytes, m = bench.build_stack(qd, si, torch, workload, DEV)
    for op in ops:
        op.y.fill_(float("nan"))
    plan = qd.StackPlan(ops, 1)
    assert plan.persistent                          # int8 body persistent, fp16 head replayed after it
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    wl = si.WORKLOADS[workload]
    names = [p for _, ms in wl.decoder.groups() for p, _, _ in ms]
    for op in ops:
        assert torch.isfinite(op.y).all()
    rng = np.random.default_rng(13)
    for name in _sample_picks(wl.decoder):
        op = ops[names.index(name)]
        fmt = "fp16" if name == "head" else wl.fmt
        assert op.w.fmt == fmt
        n, k = op.w.n, op.w.k
        rows = np.sort(rng.choice(n, 24, replace=False))
        w_rows = si.weights_torch(si.matrix_seed(wl.decoder.name, name), n, k, DEV)[rows].cpu().numpy()
        x = op.x.cpu().numpy()
        parts = _oracle_parts(fmt, w_rows)
        check_vector(_host(op.y)[rows], linear.ref_linear(fmt, parts, x), linear.row_max_abs(fmt, parts),
                     x, f"{name} ({fmt})")
    plan.close()


@pytest.mark.parametrize("m,fmt", [(1, "int8_b32"), (16, "int8_b32"), (16, "int4_g64")])
def test_plan_wait_timeout_reported_and_recovers(qd, m, fmt):
    """The persistent kernel's waits are bounded.  With the bound set to no
    polls from the host, waits time out: the run still ends, the error word
    reports it, and the plan resets its scratch; with the default bound
    restored the next run is correct (oracle parity on a chained step)."""
    from int4_quantized_decode_amd import LinearOp
    k = 1024
    ws = [si.weights(si.seed_for("timeout-w", g), k, k) for g in range(3)]
    x0 = si.activations(si.seed_for("timeout-x", m), m, k)
    shape = (m, k) if m > 1 else (k,)
    ys = [torch.empty(shape, dtype=torch.float16, device=DEV) for _ in range(3)]
    xs = [_gpu(x0.reshape(shape)), ys[0], ys[1]]
    ops = [LinearOp(_pack(qd, fmt, _gpu(w)), xs[g], ys[g], g) for g, w in enumerate(ws)]
    plan = qd.StackPlan(ops, m)
    assert plan.persistent
    plan.set_spin_limit(0)
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() != 0
    plan.set_spin_limit(1 << 20)
    for y in ys:
        y.fill_(float("nan"))
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    x = x0.astype(np.float64)
    for g, w in enumerate(ws):
        parts = _oracle_parts(fmt, w)
        Y = _host(ys[g]).reshape(m, k)
        Y_ref = linear.ref_linear(fmt, parts, x).reshape(m, k)
        for t in range(m):
            check_vector(Y[t], Y_ref[t], linear.row_max_abs(fmt, parts), x[t], f"group {g} token {t}")
        x = Y.astype(np.float64)
    plan.close()


@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
def test_plan_multi_token_longest_k(qd, fmt):
    """The 16-token persistent step at the longest K the packers accept
    (K = 24576, 96 super-blocks: exactly the per-workgroup tile budget, one
    row-group per workgroup, so 263 row-groups split into two row ranges),
    against the oracle on every token row, and repeated runs bit-identical.
    Every valid K therefore fits that budget."""
    from int4_quantized_decode_amd import LinearOp
    m, n, k = 16, 4200, 24576
    w = si.weights(si.seed_for("longk-w", k), n, k)
    X = si.activations(si.seed_for("longk-x", k), m, k)
    y = torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
    plan = qd.StackPlan([LinearOp(_pack(qd, fmt, _gpu(w)), _gpu(X), y, 0)], m)
    assert plan.persistent
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    Y = _host(y).copy()
    y.fill_(float("nan"))
    plan.run()
    torch.cuda.synchronize()
    assert np.array_equal(_host(y).view(np.uint16), Y.view(np.uint16))
    parts = _oracle_parts(fmt, w)
    Y_ref = linear.ref_linear(fmt, parts, X)
    rmax = linear.row_max_abs(fmt, parts)
    for t in range(m):
        check_vector(Y[t], Y_ref[t], rmax, X[t], f"K={k} token {t}")
    plan.close()


@pytest.mark.parametrize("m", [1, 4])
def test_plan_persistent_prefix_and_replayed_tail(qd, m):
    """A step whose first group qualifies for the persistent kernel and whose
    later groups do not all qualify: int8 -> fp16 -> int8, each group reading
    the one before it.  The plan runs the first group persistently and
    replays the other two after it; each output matches the oracle on the
    fp16 input the device produced, and repeated runs are bit-identical."""
    from int4_quantized_decode_amd import LinearOp
    k0, n0, n1, n2 = 1024, 2048, 1536, 640
    w0 = si.weights(si.seed_for("tail-w0"), n0, k0)
    w1 = si.weights(si.seed_for("tail-w1"), n1, n0)
    w2 = si.weights(si.seed_for("tail-w2"), n2, n1)
    x0 = si.activations(si.seed_for("tail-x0", m), m, k0)
    shape = (lambda n: (m, n) if m > 1 else (n,))
    ys = [torch.full(shape(n), float("nan"), dtype=torch.float16, device=DEV) for n in (n0, n1, n2)]
    ops = [LinearOp(qd.qpack_int8_b32(_gpu(w0)), _gpu(x0.reshape(shape(k0))), ys[0], 0),
           LinearOp(qd.qpack_fp16(_gpu(w1)), ys[0], ys[1], 1),
           LinearOp(qd.qpack_int8_b32(_gpu(w2)), ys[1], ys[2], 2)]
    plan = qd.StackPlan(ops, m)
    assert plan.persistent
    first = None
    for rep in range(3):
        for y in ys:
            y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        outs = [_host(y).reshape(m, -1).copy() for y in ys]
        if first is None:
            first = outs
        else:
            for a_, b_ in zip(first, outs):
                assert np.array_equal(a_.view(np.uint16), b_.view(np.uint16))
    xs = [x0, first[0].astype(np.float64), first[1].astype(np.float64)]
    for i, (fmt, w) in enumerate((("int8_b32", w0), ("fp16", w1), ("int8_b32", w2))):
        parts = _oracle_parts(fmt, w)
        Y_ref = linear.ref_linear(fmt, parts, xs[i]).reshape(m, -1)
        for t in range(m):
            check_vector(first[i][t], Y_ref[t], linear.row_max_abs(fmt, parts), xs[i][t], f"group {i} token {t}")
    plan.close()


@pytest.mark.parametrize("fmt", FMTS)
def test_plan_multi_token_groups(qd, fmt):
    """A plan at m > 1 (int8 and INT4: the persistent kernel; fp16: it replays
    the per-group launches): groups of many shapes (K = 1088, a ragged
    super-block tail; 4096 x 4096; K = 12288; a fused pair; a group large
    enough for multi-row-group workgroups) and m below 16.  Runs repeat with
    outputs poisoned in between and are bit-identical; a replaying plan's
    outputs equal decode_linear_stack's."""
    from int4_quantized_decode_amd import LinearOp
    shapes = [("a", [(200, 1088), (72, 1088)]), ("b", [(4096, 4096)]), ("c", [(512, 12288)]),
              ("d", [(16400, 2048)])]
    for m in (16, 5):
        ops, meta = [], []
        for gid, (gname, mems) in enumerate(shapes):
            k = mems[0][1]
            X = si.activations(si.seed_for("splitk-x", gname, m), m, k)
            xg = _gpu(X)
            for i, (n, kk) in enumerate(mems):
                w = si.weights(si.seed_for("splitk-w", gname, i), n, kk)
                y = torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
                ops.append(LinearOp(_pack(qd, fmt, _gpu(w)), xg, y, gid))
                meta.append((f"{gname}{i}", w, X))
        plan = qd.StackPlan(ops, m)
        assert plan.persistent == (fmt != "fp16")
        first = None
        for rep in range(3):
            for op in ops:
                op.y.fill_(float("nan"))
            plan.run()
            outs = [_host(op.y).copy() for op in ops]
            if first is None:
                first = outs
                for Y, (name, w, X) in zip(outs, meta):
                    parts = _oracle_parts(fmt, w)
                    Y_ref = linear.ref_linear(fmt, parts, X)
                    rmax = linear.row_max_abs(fmt, parts)
                    for t in range(m):
                        check_vector(Y[t], Y_ref[t], rmax, X[t], f"{fmt} {name} m={m} token {t}")
            else:
                for a_, b_ in zip(first, outs):
                    assert np.array_equal(a_.view(np.uint16), b_.view(np.uint16))
        if not plan.persistent:
            # the same launches as decode_linear_stack: the same bytes
            for op in ops:
                op.y.fill_(float("nan"))
            qd.decode_linear_stack(ops, m)
            for op, Yp in zip(ops, first):
                assert np.array_equal(_host(op.y).view(np.uint16), Yp.view(np.uint16))
        assert plan.error() == 0
        plan.close()


@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
def test_plan_multi_token_split_and_chain(qd, fmt):
    """The persistent kernel at m > 1: a group too large for one range of
    tile partials per workgroup is split into row ranges (a member crossing
    the split, a ragged last row-group), a group reads an earlier group's
    output (activation blocks read only after the boundary), and a later
    group reads a member of the split group.  Oracle parity per token row,
    with each dependent input taken from the plan's own fp16 output, and
    bit-identical repeats, at m = 16 and m = 3."""
    from int4_quantized_decode_amd import LinearOp
    shapes = {"a": (4096, 1024), "b": (1000, 4096), "c0": (5056, 12288), "c1": (4010, 12288),
              "d": (600, 5056)}
    ws = {name: si.weights(si.seed_for("split-w", name), n, k) for name, (n, k) in shapes.items()}
    parts = {name: _oracle_parts(fmt, w) for name, w in ws.items()}
    pws = {name: _pack(qd, fmt, _gpu(w)) for name, w in ws.items()}
    for m in (16, 3):
        xa = si.activations(si.seed_for("split-xa", m), m, 1024)
        xc = si.activations(si.seed_for("split-xc", m), m, 12288)
        y = {name: torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
             for name, (n, _) in shapes.items()}
        xa_g, xc_g = _gpu(xa), _gpu(xc)
        ops = [LinearOp(pws["a"], xa_g, y["a"], 0),
               LinearOp(pws["b"], y["a"], y["b"], 1),          # reads group 0's output
               LinearOp(pws["c0"], xc_g, y["c0"], 2),          # split into row ranges
               LinearOp(pws["c1"], xc_g, y["c1"], 2),
               LinearOp(pws["d"], y["c0"], y["d"], 3)]          # reads a member of the split group
        plan = qd.StackPlan(ops, m)
        assert plan.persistent
        first = None
        for rep in range(3):
            for t in y.values():
                t.fill_(float("nan"))
            plan.run()
            torch.cuda.synchronize()
            assert plan.error() == 0
            outs = {name: _host(t).copy() for name, t in y.items()}
            if first is None:
                first = outs
            else:
                for name in outs:
                    assert np.array_equal(first[name].view(np.uint16), outs[name].view(np.uint16)), name
        inputs = {"a": xa, "b": first["a"].astype(np.float64), "c0": xc, "c1": xc,
                  "d": first["c0"].astype(np.float64)}
        for name in shapes:
            Y_ref = linear.ref_linear(fmt, parts[name], inputs[name])
            rmax = linear.row_max_abs(fmt, parts[name])
            for t in range(m):
                check_vector(first[name][t], Y_ref[t], rmax, inputs[name][t], f"{name} m={m} token {t}")
        plan.close()


@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
def test_plan_multi_token_unit_across_members(qd, fmt):
    """At m > 1 each workgroup takes its row-groups two at a time (a unit at
    one super-block), and a unit may hold the last row-group of one member
    and the first of the next.  Each of its tiles must come from its own
    member's weights, also when the members' blobs are not adjacent in
    memory (a spacer buffer between them here).  Members with odd row-group
    counts and ragged last row-groups, K spanning several super-blocks with
    a ragged tail; oracle parity per token at m = 16 and 3."""
    from int4_quantized_decode_amd import LinearOp
    K = 1088
    shapes = [(4075, K), (1000, K), (1613, K)]          # 255 + 63 + 101 row-groups
    ws = [si.weights(si.seed_for("unit-w", fmt, i), n, k) for i, (n, k) in enumerate(shapes)]
    pws, spacers = [], []
    for w in ws:
        pws.append(_pack(qd, fmt, _gpu(w)))
        spacers.append(torch.empty(1 << 20, dtype=torch.uint8, device=DEV))
    for m in (16, 3):
        x = si.activations(si.seed_for("unit-x", fmt, m), m, K)
        x_g = _gpu(x)
        ys = [torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV) for n, _ in shapes]
        ops = [LinearOp(pw, x_g, y, 0) for pw, y in zip(pws, ys)]
        v, groups, members, sched = _plan_tables(qd, ops, m)
        G, ng, nm = v[8], v[6], v[7]
        assert v[1] == 1 and ng == 1 and nm == 3
        starts = {mb[3] for mb in members[1:]}                          # members' first row-groups
        sched = sched[:G]
        crossing = sum(1 for _, _, rg0, nseg in sched for u in range(0, nseg - 1, 2) if rg0 + u + 1 in starts)
        assert crossing >= 1, "no unit holds row-groups of two members"
        plan = qd.StackPlan(ops, m)
        assert plan.persistent
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        for i, (w, y) in enumerate(zip(ws, ys)):
            parts = _oracle_parts(fmt, w)
            Y_ref = linear.ref_linear(fmt, parts, x)
            rmax = linear.row_max_abs(fmt, parts)
            got = _host(y)
            for t in range(m):
                check_vector(got[t], Y_ref[t], rmax, x[t], f"{fmt} member {i} m={m} token {t}")
        plan.close()
    del spacers


def test_plan_multi_token_copy_of_a_split_member(qd):
    """At m > 1 an op whose whole output is a later group's activation also
    writes it in matrix-core order, and a group split into row ranges
    addresses its part of that copy by an offset.  Group 0's second member
    starts 4 row-groups in, so the split (every 1024 row-groups at K = 5120
    on 256 workgroups) cuts it inside a 256-row block: it writes no copy and
    group 1 reads its activation in place.  Group 2's first member is cut at
    a whole block and keeps its copy, both slices writing it, and group 3
    reads it.  The schedule is checked on the host, then the step's outputs:
    the consumers in full, the producers on sampled rows around and away
    from the cut, against the oracle."""
    from int4_quantized_decode_amd import LinearOp
    m, fmt = 16, "int8_b32"
    shapes = {"a": (64, 5120), "b": (24576, 5120), "c": (512, 24576),
              "d": (24576, 5120), "e": (64, 5120), "f": (512, 24576)}
    ws = {name: si.weights(si.seed_for("cut-w", name), n, k) for name, (n, k) in shapes.items()}
    pws = {name: _pack(qd, fmt, _gpu(w)) for name, w in ws.items()}
    x = si.activations(si.seed_for("cut-x", m), m, 5120)
    x_g = _gpu(x)
    y = {name: torch.full((m, n), float("nan"), dtype=torch.float16, device=DEV)
         for name, (n, _) in shapes.items()}
    ops = [LinearOp(pws["a"], x_g, y["a"], 0), LinearOp(pws["b"], x_g, y["b"], 0),
           LinearOp(pws["c"], y["b"], y["c"], 1),
           LinearOp(pws["d"], x_g, y["d"], 2), LinearOp(pws["e"], x_g, y["e"], 2),
           LinearOp(pws["f"], y["d"], y["f"], 3)]
    # The schedule this device gets: b's slices carry no copy, d's do.
    v, groups, members, _ = _plan_tables(qd, ops, m)
    ng, nm = v[6], v[7]
    yptr = {name: t.data_ptr() for name, t in y.items()}
    if v[8] != 256:
        pytest.skip("the cuts are laid out for 256 compute units")
    assert v[1] == 1 and ng == 6                                  # persistent, groups 0 and 2 split
    in_y = lambda p, name: yptr[name] <= p < yptr[name] + shapes[name][0] * 2
    assert [mb[6] for mb in members if in_y(mb[1], "b")] == [-1, -1]
    d_copies = [mb[6] for mb in members if in_y(mb[1], "d")]
    assert len(d_copies) == 2 and min(d_copies) >= 0 and d_copies[1] - d_copies[0] == 1024 * 512
    assert groups[[g[0] for g in groups].index(yptr["b"])][9] == -1      # c reads in place
    assert groups[[g[0] for g in groups].index(yptr["d"])][9] >= 0       # f reads d's copy

    plan = qd.StackPlan(ops, m)
    assert plan.persistent
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    out = {name: _host(t).copy() for name, t in y.items()}
    for name, src in (("c", "b"), ("f", "d")):
        parts = _oracle_parts(fmt, ws[name])
        xin = out[src].astype(np.float64)
        Y_ref = linear.ref_linear(fmt, parts, xin)
        rmax = linear.row_max_abs(fmt, parts)
        for t in range(m):
            check_vector(out[name][t], Y_ref[t], rmax, xin[t], f"{name} token {t}")
    rng = np.random.default_rng(si.seed_for("cut-rows"))
    for name in ("a", "b", "d", "e"):
        N = shapes[name][0]
        rows = np.unique(np.concatenate([np.arange(min(N, 48)), np.arange(max(0, N - 48), N),
                                         np.arange(16256, 16448) % N, rng.integers(0, N, 200)]))
        parts = _oracle_parts(fmt, ws[name][rows])
        Y_ref = linear.ref_linear(fmt, parts, x)
        rmax = linear.row_max_abs(fmt, parts)
        for t in range(m):
            check_vector(out[name][t][rows], Y_ref[t], rmax, x[t], f"{name} token {t}")
    plan.close()


def _group_slices(ops):
    """[(first op, end op)] of each group of consecutive equal `group` ids."""
    out, i = [], 0
    while i < len(ops):
        e = i + 1
        while e < len(ops) and ops[e].group == ops[i].group:
            e += 1
        out.append((i, e))
        i = e
    return out


def _plan_tables(qd, ops, m):
    """qd_stack_plan_describe's words for `ops` on this device, cut into the
    header, the group records (12 words), the member records (8 words) and
    the per-workgroup schedule entries (4 words, group-major)."""
    v = qd.describe_stack_plan(ops, m)
    assert v[0] == 4
    ng, nm, G = v[6], v[7], v[8]
    groups = [v[22 + 12 * i:34 + 12 * i] for i in range(ng)]
    mo = 22 + 12 * ng
    members = [v[mo + 8 * i:mo + 8 * i + 8] for i in range(nm)]
    so = mo + 8 * nm
    sched = [v[so + 4 * i:so + 4 * i + 4] for i in range(ng * G)]
    return v, groups, members, sched


def _prefix_states(qd, ops, m, restore, snapshot):
    """The buffers before the step and after each of its groups, from plans of
    the step's first 1, 2, ... groups, each run from the same initial state.
    A group's schedule is the same in every plan that holds it (its ranges
    depend on its own row-groups only), so its outputs are bit-identical
    across them."""
    states = []
    restore()
    torch.cuda.synchronize()
    states.append(snapshot())
    for _, e in _group_slices(ops):
        sub = qd.StackPlan(ops[:e], m)
        assert sub.persistent
        restore()
        sub.run()
        torch.cuda.synchronize()
        assert sub.error() == 0
        states.append(snapshot())
        sub.close()
    return states


@pytest.mark.parametrize("m,packed,fmt", [(1, False, "int8_b32"), (1, True, "int8_b32"), (16, False, "int8_b32"),
                                          (16, True, "int8_b32"), (16, False, "int4_g64"), (16, True, "int4_g64")])
def test_plan_buffer_orderings(qd, m, packed, fmt):
    """The persistent step orders each boundary from the step's buffers: an
    input no earlier output overlaps is staged early, one that an earlier
    output overlaps (not only the previous group's) only after the barrier,
    through the caches only when no earlier access can have left a stale
    copy of its cache lines; outputs a later group reads or rewrites are
    stored before the stamp.  Checked against a sequential model of the
    buffers: a group reading the output of two groups back, a group
    rewriting an earlier group's output (the later value must win), a group
    overwriting an earlier group's input that a later group then reads, and
    independent groups between them.  Separate buffers, and buffers packed
    16 bytes apart in one allocation (neighbours share cache lines); one and
    16 token rows."""
    from int4_quantized_decode_amd import LinearOp
    k = 1024
    nbuf = 6
    shape = (m, k) if m > 1 else (k,)
    if packed:
        big = torch.empty(nbuf * (m * k + 8), dtype=torch.float16, device=DEV)
        bufs = [big[i * (m * k + 8):i * (m * k + 8) + m * k].view(shape) for i in range(nbuf)]
    else:
        bufs = [torch.empty(shape, dtype=torch.float16, device=DEV) for _ in range(nbuf)]
    init = [si.activations(si.seed_for("order-buf", i, m), m, k).reshape(shape) for i in range(nbuf)]
    # (x buffer, y buffer) per group, in step order; all matrices are k x k
    prog = [(0, 1),   # g0: independent input
            (2, 3),   # g1: independent (early staging)
            (1, 4),   # g2: reads g0's output, two groups back
            (5, 3),   # g3: rewrites g1's output
            (4, 0),   # g4: reads g2's output, overwrites g0's input
            (0, 2),   # g5: reads g4's output from g0's old input buffer
            (3, 5)]   # g6: reads g3's rewrite of buffer 3
    ws = [si.weights(si.seed_for("order-w", g), k, k) for g in range(len(prog))]
    pws = [_pack(qd, fmt, _gpu(w)) for w in ws]
    ops = [LinearOp(pws[g], bufs[xb], bufs[yb], g) for g, (xb, yb) in enumerate(prog)]
    plan = qd.StackPlan(ops, m)
    assert plan.persistent

    def restore():
        for i, b in enumerate(bufs):
            b.copy_(_gpu(init[i]))

    def snapshot():
        return [_host(b).copy() for b in bufs]

    # Each group against the oracle on the input the device gave it, at the
    # acceptance bound; every other buffer untouched by it.
    states = _prefix_states(qd, ops, m, restore, snapshot)
    for g, (xb, yb) in enumerate(prog):
        parts = _oracle_parts(fmt, ws[g])
        xin = states[g][xb].reshape(m, k)
        assert np.all(np.isfinite(xin.astype(np.float64))), f"group {g} input"
        ref = linear.ref_linear(fmt, parts, xin)
        got = states[g + 1][yb].reshape(m, k)
        rmax = linear.row_max_abs(fmt, parts)
        for t in range(m):
            check_vector(got[t], ref[t], rmax, xin[t], f"buffer {yb} (group {g}) token {t}")
        for b in range(nbuf):
            if b != yb:
                assert np.array_equal(states[g + 1][b].view(np.uint16), states[g][b].view(np.uint16)), \
                    f"group {g} changed buffer {b}"
    # The whole step in one plan, three runs: exactly the sequence above.
    for rep in range(3):
        restore()
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        for b_, (a_, want_) in enumerate(zip(snapshot(), states[-1])):
            assert np.array_equal(a_.view(np.uint16), want_.view(np.uint16)), f"rep {rep} buffer {b_}"
    plan.close()


def test_plan_random_steps_against_sequential_model(qd):
    """Random steps run as persistent plans against a sequential model of the
    buffers built from the oracle: groups of 1-3 members in one fp16 arena;
    each group reads a fresh region, an earlier op's whole output or (one
    token row) a slice of one; outputs go to fresh regions or overwrite an
    earlier op's output.  Plans of the step's first groups give the arena
    after each group: every group's outputs against the oracle on the input
    the device gave it, at the acceptance bound, and the one-plan step must
    reproduce the final arena bit for bit."""
    from int4_quantized_decode_amd import LinearOp
    rng = np.random.default_rng(si.seed_for("random-steps"))
    arena_n = 1 << 21
    for case in range(24):
        fmt = ["int8_b32", "int4_g64"][case % 2]
        m = [1, 5, 16][(case // 2) % 3]
        init = si.activations(si.seed_for("random-arena", case), 1, arena_n)[0]
        arena = _gpu(init)
        top = 0

        def take(n):
            nonlocal top
            off = top
            top += (n + 63) // 64 * 64
            assert top <= arena_n
            return off

        ops, prog, outs = [], [], []
        for g in range(int(rng.integers(2, 7))):
            k = int(rng.choice([256, 512, 1024, 1088]))
            cands = [(o, n) for o, n in outs if (n == k or (m == 1 and n >= k))]
            if cands and rng.random() < 0.6:
                o, n = cands[int(rng.integers(len(cands)))]
                xo = o + (8 * int(rng.integers(0, (n - k) // 8 + 1)) if m == 1 else 0)
            else:
                xo = take(m * k)
            members = []
            for _ in range(int(rng.integers(1, 4))):
                n = int(rng.choice([16, 48, 100, 256, 1000, 1088]))
                same = [o for o, nn in outs if nn == n and not (o < xo + m * k and xo < o + m * n)
                        and all(o != mo for mo, _, _ in members)]
                yo = same[0] if same and rng.random() < 0.25 else take(m * n)
                w = si.weights(si.seed_for("random-w", case, g, len(members)), n, k)
                members.append((yo, n, w))
            for yo, n, w in members:
                ops.append(LinearOp(_pack(qd, fmt, _gpu(w)), arena[xo:xo + m * k].view(m, k) if m > 1
                                    else arena[xo:xo + k], arena[yo:yo + m * n].view(m, n) if m > 1
                                    else arena[yo:yo + n], g))
            prog.append((xo, k, members))
            outs.extend((yo, n) for yo, n, _ in members)
        plan = qd.StackPlan(ops, m)
        assert plan.persistent, f"case {case}"
        init_g = _gpu(init)

        def restore():
            arena.copy_(init_g)

        def snapshot():
            return _host(arena).copy()

        # Each group against the oracle on the input the device gave it, at
        # the acceptance bound, and nothing outside its outputs changed; then
        # the whole step in one plan must reproduce the final state exactly.
        states = _prefix_states(qd, ops, m, restore, snapshot)
        for g, (xo, k, members) in enumerate(prog):
            X = states[g][xo:xo + m * k].reshape(m, k)
            assert np.all(np.isfinite(X.astype(np.float64))), f"case {case} group {g} input"
            touched = np.zeros(arena_n, bool)
            for yo, n, w in members:
                parts = _oracle_parts(fmt, w)
                Y = linear.ref_linear(fmt, parts, X)
                G_ = states[g + 1][yo:yo + m * n].reshape(m, n)
                rmax = linear.row_max_abs(fmt, parts)
                for t in range(m):
                    check_vector(G_[t], Y[t], rmax, X[t], f"case {case} ({fmt}, m={m}) group {g} output at {yo} token {t}")
                touched[yo:yo + m * n] = True
            assert np.array_equal(states[g + 1][~touched].view(np.uint16), states[g][~touched].view(np.uint16)), \
                f"case {case} group {g} wrote outside its outputs"
        restore()
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        assert np.array_equal(snapshot().view(np.uint16), states[-1].view(np.uint16)), f"case {case}"
        plan.close()


def _one_row_per_row_group(n, salt):
    """One row of every 16-row row-group, at a position that moves from
    row-group to row-group (every row lane is used)."""
    r = np.arange((n + 15) // 16)
    return np.minimum(16 * r + (7 * r + salt) % 16, n - 1)


@pytest.mark.parametrize("workload", ["qwen3-8b-int8-m1", "qwen3-8b-int8-chain-m1", "qwen3-8b-int4-m1",
                                      "qwen3-8b-int8-m16", "qwen3.8-27b-int8-m1"])
def test_plan_full_size_every_row_group(qd, workload):
    """The 8B-shaped step as the bench times it (and its chained, INT4 and
    16-token variants): one row of every row-group of every projection
    against the oracle, every token row, on the activations the op read."""
    import bench
    ops, alg_bytes, weight_bytes, m = bench.build_stack(qd, si, torch, workload, DEV)
    plan = qd.StackPlan(ops, m)
    assert plan.persistent
    for op in ops:
        op.y.fill_(float("nan"))
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    wl = si.WORKLOADS[workload]
    names = [p for _, ms in wl.decoder.groups() for p, _, _ in ms]
    assert len(names) == len(ops)
    for i, (name, op) in enumerate(zip(names, ops)):
        n, k = op.w.n, op.w.k
        rows = _one_row_per_row_group(n, i)
        w_full = si.weights_torch(si.matrix_seed(wl.decoder.name, name), n, k, DEV)
        if wl.chain:                                   # the chained step's weight scale
            w_full.mul_(1.0 / (si.W_STD * k ** 0.5))
        w_rows = w_full[torch.from_numpy(rows).to(DEV)].cpu().numpy()
        del w_full
        x = op.x.cpu().numpy().reshape(m, k)           # the activations the op read
        parts = _oracle_parts(wl.fmt, w_rows)
        y_ref = linear.ref_linear(wl.fmt, parts, x).reshape(m, -1)
        y_got = _host(op.y).reshape(m, n)[:, rows]
        rmax = linear.row_max_abs(wl.fmt, parts)
        for t in range(m):
            check_vector(y_got[t], y_ref[t], rmax, x[t], f"{name} token {t}")
    plan.close()
    del ops
    torch.cuda.empty_cache()


# every matrix of every configuration: (model name, format, workload holding it)
PACK_CONFIGS = [("single", "int8_b32", "gemv-2048x2048-int8"), ("qwen3-2b", "int8_b32", "qwen3-2b-int8-m1"),
                ("qwen3-4b", "int8_b32", "qwen3-4b-int8-m1"), ("qwen3-8b", "int8_b32", "qwen3-8b-int8-m1"),
                ("qwen3-8b", "int4_g64", "qwen3-8b-int4-m1"), ("qwen3.8-27b", "int8_b32", "qwen3.8-27b-int8-m1"),
                ("qwen3-2b", "fp16", "qwen3-2b-int8-fp16head-m1")]


@pytest.mark.parametrize("model,fmt,workload", PACK_CONFIGS)
def test_pack_every_matrix_sampled(qd, model, fmt, workload):
    """Every matrix of every configuration packed on the device: the first,
    the last and two random row-groups of each compared byte for byte with
    the oracle's blob of those rows (a row-group's tiles are contiguous, so
    its bytes are the blob of its 16 rows).  The fp16 case is the int8lin
    head."""
    wl = si.WORKLOADS[workload]
    if wl.single is not None:
        mats = [("W", *wl.single)]
    else:
        mats = [(p, n, k) for _, ms in wl.decoder.groups() for p, n, k in ms]
        if fmt == "fp16":
            mats = [mt for mt in mats if mt[0] == "head"]
    rng = np.random.default_rng(si.seed_for("pack-every", model, fmt))
    tile = {"int8_b32": 4352, "int4_g64": 2304, "fp16": 8192}[fmt]
    for name, n, k in mats:
        w_full = si.weights_torch(si.matrix_seed(model, name), n, k, DEV)
        blob = _pack(qd, fmt, w_full).blob
        R, J = (n + 15) // 16, (k + 255) // 256
        picks = sorted({0, R - 1, *(int(v) for v in rng.integers(0, R, 2))})
        for r in picks:
            rows = torch.arange(16 * r, min(n, 16 * r + 16), device=DEV)
            w_rows = w_full[rows].cpu().numpy()
            want = _oracle_blob(fmt, _oracle_parts(fmt, w_rows))
            got = blob[r * J * tile:(r + 1) * J * tile].cpu().numpy()
            assert want.size == got.size == J * tile
            diff = np.flatnonzero(got != want)
            assert diff.size == 0, f"{model} {fmt} {name} row-group {r}: {diff.size} bytes differ"
        del w_full, blob
    torch.cuda.empty_cache()


@pytest.mark.parametrize("m", [1, 16])
def test_plan_new_activations_every_step(qd, m):
    """One plan run for several decode steps, with fresh activations written
    into the step's input buffer before each (as a decoder does token after
    token).  The paths that read activations through the caches must see
    this step's values, not lines left from the last one: at one token row a
    chained group read through the caches (order flag 8); at 16 token rows an
    activation copied into matrix-core order before the step and one written
    in that order by the op producing it.  The schedule is asserted to take
    those paths; every op of every step is checked against the oracle on
    the input the device read, at the acceptance bound."""
    from int4_quantized_decode_amd import LinearOp
    k = 1024
    shape = (lambda n: (m, n) if m > 1 else (n,))
    ws = [si.weights(si.seed_for("steps-w", m, i), k, k) for i in range(4)]
    parts = [quant.quantize_int8_b32(w) for w in ws]
    pws = [qd.qpack_int8_b32(_gpu(w)) for w in ws]
    bufs = [torch.zeros(shape(k), dtype=torch.float16, device=DEV) for _ in range(len(ws) + 1)]
    ops = [LinearOp(pws[i], bufs[i], bufs[i + 1], i) for i in range(len(ws))]
    v, groups, members, _ = _plan_tables(qd, ops, m)
    ng, nm, njobs = v[6], v[7], v[10]
    assert v[1] == 1 and ng == len(ws)
    if m == 1:
        assert all(g[8] & 8 for g in groups[1:]), "chained groups should read through the caches"
    else:
        assert njobs >= 1 and groups[0][9] >= 0, "no pre-step copy of the step's input"
        assert all(g[9] >= 0 for g in groups[1:]), "chained groups should read producer-written copies"
        assert all(mb[6] >= 0 for mb in members[:-1]), "producers should write their outputs' copies"
    plan = qd.StackPlan(ops, m)
    assert plan.persistent
    for step in range(5):
        x = si.activations(si.seed_for("steps-x", m, step), m, k).reshape(shape(k))
        bufs[0].copy_(_gpu(x))
        for b in bufs[1:]:
            b.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        vals = [_host(b).reshape(m, k).copy() for b in bufs]
        assert np.array_equal(vals[0].view(np.uint16), x.reshape(m, k).view(np.uint16))
        for i in range(len(ws)):
            assert np.all(np.isfinite(vals[i].astype(np.float64))), f"step {step} op {i} input"
            y_ref = linear.ref_linear("int8_b32", parts[i], vals[i])
            rmax = linear.row_max_abs("int8_b32", parts[i])
            for t in range(m):
                check_vector(vals[i + 1][t], y_ref[t], rmax, vals[i][t], f"step {step} op {i} token {t}")
    plan.close()


DYNAMIC = 64          # qd_stack_plan_describe order flag: the last group is split at run time


@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
@pytest.mark.parametrize("chained", [False, True])
def test_plan_dynamic_last_group(qd, fmt, chained):
    """The step's last group split at run time (workgroups claim chunks of
    row-groups from a device counter), which a plan does from 3 GiB of
    weights: groups of copies of one 32768 x 16384 matrix make up the
    bytes.  The last group has two members with ragged row tails
    (200003 and 62424 rows, 16403 row-groups: chunks of 2, the last one half
    past the group) and K = 2304 (9 super-blocks: an INT4 hand-out of two
    holds a missing tile at the end of each row-group); it reads an
    activation of its own, or the output of the group before it (chained):
    then it waits for that group, and a step with such a wait keeps the
    fixed split, which the same checks cover.  Three runs with fresh
    activations (the claim counter alternates between runs):
    one row of every row-group and every row of the members' last two
    row-groups against the oracle on the inputs the device read; a rerun on
    the same input bit-identical; the no-allocation entry point
    bit-identical too."""
    from int4_quantized_decode_amd import LinearOp
    k = 2304
    pack = _pack_fn(qd, fmt)
    nf, kf = 32768, 16384
    wf = si.weights_torch(si.seed_for("dyn-filler", fmt), nf, kf, DEV)
    pf = pack(wf)
    frows = np.sort(np.random.default_rng(si.seed_for("dyn-filler-rows", fmt)).choice(nf, 48, replace=False))
    parts_f = _oracle_parts(fmt, wf[torch.from_numpy(frows).to(DEV)].cpu().numpy())
    del wf
    copies = -(-(6 << 30) // pf.blob.numel())
    xf = _gpu(si.activations(si.seed_for("dyn-xf", fmt), 1, kf)[0])
    ops = [LinearOp(pf, xf, torch.zeros(nf, dtype=torch.float16, device=DEV), i) for i in range(copies)]
    w0 = si.weights(si.seed_for("dyn-w0", fmt), k, k)
    parts0 = _oracle_parts(fmt, w0)
    x0 = torch.zeros(k, dtype=torch.float16, device=DEV)
    y0 = torch.zeros(k, dtype=torch.float16, device=DEV)
    x1 = y0 if chained else torch.zeros(k, dtype=torch.float16, device=DEV)
    ops.append(LinearOp(pack(_gpu(w0)), x0, y0, copies))
    heads = []
    for i, n in enumerate((200003, 62424)):
        w = si.weights_torch(si.seed_for("dyn-w", fmt, i), n, k, DEV)
        y = torch.zeros(n, dtype=torch.float16, device=DEV)
        ops.append(LinearOp(pack(w), x1, y, copies + 1))
        rows = _one_row_per_row_group(n, i)
        rows = np.unique(np.concatenate([rows, np.arange(max(0, n - 32), n)]))
        w_rows = w[torch.from_numpy(rows).to(DEV)].cpu().numpy()
        del w
        heads.append((n, y, rows, _oracle_parts(fmt, w_rows)))
    v, groups, _, sched = _plan_tables(qd, ops, 1)
    G = v[8]
    assert v[1] == 1 and len(groups) == copies + 2
    assert bool(groups[-1][8] & DYNAMIC) == (not chained)
    assert not any(g[8] & DYNAMIC for g in groups[:-1])
    if not chained:
        R = -(-200003 // 16) + -(-62424 // 16)
        assert G == 256 and R == 16403
        assert v[18] == max(1, R // (32 * G)) == 2 and v[20] == -(-R // 2), "chunk size / chunk count"
        assert all(sc[0] == 0 and sc[3] == 0 for sc in sched[(copies + 1) * G:])
    plan = qd.StackPlan(ops, 1)
    assert plan.persistent
    xfh = _host(xf)
    outs = []
    for step in range(3):
        x = si.activations(si.seed_for("dyn-x", fmt, chained, step), 1, k)[0]
        x0.copy_(_gpu(x))
        if not chained:
            x1.copy_(_gpu(si.activations(si.seed_for("dyn-x1", fmt, step), 1, k)[0]))
        for op in ops:
            op.y.fill_(float("nan"))
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        yf = [_host(op.y) for op in ops[:copies]]
        assert all(np.array_equal(yf[0].view(np.uint16), a.view(np.uint16)) for a in yf[1:])
        check_vector(yf[0][frows], linear.ref_linear(fmt, parts_f, xfh), linear.row_max_abs(fmt, parts_f), xfh,
                     f"step {step} filler")
        y0h, x1h = _host(y0).copy(), _host(x1).copy()
        check_vector(y0h, linear.ref_linear(fmt, parts0, x), linear.row_max_abs(fmt, parts0), x, f"step {step} A")
        for i, (n, y, rows, parts) in enumerate(heads):
            yh = _host(y)
            assert np.all(np.isfinite(yh.astype(np.float64))), f"step {step} member {i}: unwritten rows"
            check_vector(yh[rows], linear.ref_linear(fmt, parts, x1h), linear.row_max_abs(fmt, parts), x1h,
                         f"step {step} member {i}")
        outs = [_host(op.y).copy() for op in ops[copies:]]
    plan.run()                                     # the same input again: the same bits
    torch.cuda.synchronize()
    assert plan.error() == 0
    for a, op in zip(outs, ops[copies:]):
        assert np.array_equal(a.view(np.uint16), _host(op.y).view(np.uint16))
    plan.close()
    err = torch.zeros(1, dtype=torch.int32, device=DEV)
    for op in ops:
        op.y.fill_(float("nan"))
    qd.stack_run_noalloc(ops, 1, err)
    torch.cuda.synchronize()
    assert int(err.item()) == 0
    for a, op in zip(outs, ops[copies:]):
        assert np.array_equal(a.view(np.uint16), _host(op.y).view(np.uint16)), "no-allocation step differs"
    del ops, heads, pf
    torch.cuda.empty_cache()
