"""GPU parity of the fused glue: the RMSNorm and gated-product prologues and
the silu epilogue of stack ops, against the oracle's glue on the same inputs.

Each op is checked on the activations it actually read (copied back from the
device after the run), so an error in one op cannot hide behind, or leak
into, the check of the next.  The glue's own arithmetic is checked directly
through weights that pass the glued vector through unchanged."""
import numpy as np
import pytest

import synthetic_inputs as si
from oracle import glue, linear, quant
from tests.test_gpu_parity import _plan_tables, _prefix_states
from tests.numerics import MAX_ERR_COEF, REL_L2, check_vector

torch = pytest.importorskip("torch")
pytestmark = pytest.mark.gpu

DEV = "cuda:0"
EPS = 1e-6


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


def _parts(fmt, w):
    return {"int8_b32": quant.quantize_int8_b32, "int4_g64": quant.quantize_int4_g64,
            "fp16": quant.quantize_fp16}[fmt](w)


def _pack(qd, fmt, w):
    return {"int8_b32": qd.qpack_int8_b32, "int4_g64": qd.qpack_int4_g64,
            "fp16": qd.qpack_fp16}[fmt](_gpu(w))


def _ulps(a, b):
    """|a - b| in units of the fp16 spacing at the larger magnitude.  From
    2^15 up to the largest finite value (65504) the spacing is 32; the step
    above 65504 itself would be to infinity, so the magnitude is capped at
    2^15 before taking it."""
    a64, b64 = a.astype(np.float64), b.astype(np.float64)
    big = np.minimum(np.maximum(np.abs(a64), np.abs(b64)), 32768.0).astype(np.float16)
    return np.abs(a64 - b64) / np.spacing(big).astype(np.float64)


# ------------------------------------------------------- the glue itself, exactly

def _pass_through(fmt, k):
    """A K x K weight that every format stores exactly as c * I, with c chosen
    so that c * v is exact in fp32 for fp16 v: fp16 weights hold 1; int8 b32
    blocks with one nonzero 127/128 get the exact scale 2^-7 and code 127."""
    c = 1.0 if fmt == "fp16" else 127.0 / 128.0
    return (np.eye(k, dtype=np.float32) * np.float32(c)), c


@pytest.mark.parametrize("fmt", ["int8_b32", "fp16"])
@pytest.mark.parametrize("m", [1, 3, 16])
@pytest.mark.parametrize("path", ["launches", "plan"])
def test_prologues_and_epilogue_exact(qd, fmt, m, path):
    """y = fp16(c * glued input).  The gated product is one correctly rounded
    fp16 multiply, so it must match bit for bit; RMSNorm and silu go through
    fp32 (statistic, exp, quotient), so an element may sit one fp16 step from
    the oracle's fp64 rounding, and almost none do."""
    k = 1056                                     # 4 super-blocks and a ragged tail
    w, c = _pass_through(fmt, k)
    pw = _pack(qd, fmt, w)
    x = si.activations(si.seed_for("glue-x", m), m, k)
    a = si.activations(si.seed_for("glue-a", m), m, k)
    b = si.activations(si.seed_for("glue-b", m), m, k)
    g = a.copy()
    g[0, :8] = [-65504, -20, -0.0, 20, 65504, 6e-8, -3e-5, 11.5]     # silu edge values
    gam = si.norm_weight(si.seed_for("glue-gamma"), k)
    shape = (m, k) if m > 1 else (k,)
    ab = _gpu(np.concatenate([a, b], 0).reshape(-1))                # [2, m, K]: A block then B
    xs, gs, as_ = _gpu(x.reshape(shape)), _gpu(gam), _gpu(g.reshape(shape))
    ys = [torch.full(shape, float("nan"), dtype=torch.float16, device=DEV) for _ in range(3)]
    ops = [qd.LinearOp(pw, xs, ys[0], 0, prologue="rmsnorm", gamma=gs, eps=EPS),
           qd.LinearOp(pw, ab, ys[1], 1, prologue="glu"),
           qd.LinearOp(pw, as_, ys[2], 2, epilogue="silu")]
    if path == "plan":
        plan = qd.StackPlan(ops, m)
        # the persistent kernel takes the three glued groups (fp16 steps replay): at
        # several token rows the RMSNorm factors and the gated product's copy
        # are made before the step, since no group of it writes their inputs
        assert plan.persistent == (fmt != "fp16")
        assert qd.describe_stack_plan(ops, m)[5] == (3 if fmt != "fp16" else 0)
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        plan.close()
    else:
        qd.decode_linear_stack(ops, m)
    got = [_host(y).reshape(m, k) for y in ys]

    def scaled(v16):   # fp16(c * v), exact product then one rounding
        return (v16.astype(np.float64) * c).astype(np.float16)

    want_rms = scaled(glue.rmsnorm_fp16(x, gam, EPS))
    want_glu = scaled(glue.glu_fp16(a, b))
    want_silu = glue.silu_fp16(scaled(g))
    bad = np.argwhere(got[1].view(np.uint16) != want_glu.view(np.uint16))
    assert bad.size == 0, ("gated product", len(bad), [(tuple(i), float(a[tuple(i)]), float(b[tuple(i)]),
                                                        float(got[1][tuple(i)]), float(want_glu[tuple(i)]))
                                                       for i in bad[:6]])
    for name, gv, wv in (("rmsnorm", got[0], want_rms), ("silu", got[2], want_silu)):
        d = _ulps(gv, wv)
        assert np.all(np.isfinite(gv.astype(np.float64))), name
        assert d.max() <= 1.0, (name, d.max(), np.argwhere(d > 1)[:4])
        assert np.mean(d == 0) >= 0.99, (name, np.mean(d == 0))
    # signs of zeros and the large-argument limits of silu
    assert float(got[2][0, 2]) == 0.0 and float(got[2][0, 3]) == float(want_silu[0, 3])
    assert float(got[2][0, 4]) == float(want_silu[0, 4]) and float(got[2][0, 0]) == float(want_silu[0, 0])


@pytest.mark.parametrize("m", [1, 16])
def test_glue_largest_k_sampled(qd, m):
    """The glue at the largest K (24576; the gated product reads 2 x 24576
    values per token): a weight whose row n picks one input position k_n,
    spread over all of K including its last element, so y[n] is the glued
    value at k_n scaled by 127/128 (exact, as in the pass-through test)."""
    k, n = 24576, 96
    c = 127.0 / 128.0
    ks = np.unique(np.concatenate([np.linspace(0, k - 1, n - 3).astype(int), [1, k - 2, k - 1]]))[:n]
    n = len(ks)
    w = np.zeros((n, k), np.float32)
    w[np.arange(n), ks] = np.float32(c)
    pw = _pack(qd, "int8_b32", w)
    x = si.activations(si.seed_for("glue-maxk-x", m), m, k)
    a = si.activations(si.seed_for("glue-maxk-a", m), m, k)
    b = si.activations(si.seed_for("glue-maxk-b", m), m, k)
    gam = si.norm_weight(si.seed_for("glue-maxk-g"), k)
    shape = (m, n) if m > 1 else (n,)
    ys = [torch.full(shape, float("nan"), dtype=torch.float16, device=DEV) for _ in range(3)]
    xs = _gpu(x if m > 1 else x[0])
    ab = _gpu(np.concatenate([a, b], 0).reshape(-1))
    as_ = _gpu(a if m > 1 else a[0])
    ops = [qd.LinearOp(pw, xs, ys[0], 0, prologue="rmsnorm", gamma=_gpu(gam), eps=EPS),
           qd.LinearOp(pw, ab, ys[1], 1, prologue="glu"),
           qd.LinearOp(pw, as_, ys[2], 2, epilogue="silu")]
    qd.decode_linear_stack(ops, m)
    got = [_host(y).reshape(m, n) for y in ys]

    def scaled(v16):
        return (v16.astype(np.float64) * c).astype(np.float16)

    want = [scaled(glue.rmsnorm_fp16(x, gam, EPS)[:, ks]), scaled(glue.glu_fp16(a, b)[:, ks]),
            glue.silu_fp16(scaled(a[:, ks]))]
    assert np.array_equal(got[1].view(np.uint16), want[1].view(np.uint16)), "gated product"
    for name, gv, wv in (("rmsnorm", got[0], want[0]), ("silu", got[2], want[2])):
        assert _ulps(gv, wv).max() <= 1.0, name


# ------------------------------------------------------- decoder-shaped chains

def _check_silu(s_gpu, a_ref, row_max, xin, what):
    """Stored silu outputs against silu of the oracle's unrounded product:
    |silu'| <= 1.1, so the product's bound grows by that factor, plus the
    final fp16 rounding."""
    s = s_gpu.astype(np.float64)
    want = glue.silu(a_ref)
    bound = 1.1 * MAX_ERR_COEF * float(np.linalg.norm(xin.astype(np.float64))) * row_max
    bound = bound + np.spacing(np.abs(want).astype(np.float16)).astype(np.float64)
    err = np.abs(s - want)
    bad = np.flatnonzero(err > bound)
    assert bad.size == 0, (what, bad[:8], err[bad[:4]], bound[bad[:4]])
    nrm = float(np.linalg.norm(want))
    if nrm:
        assert float(np.linalg.norm(s - want)) / nrm <= 2 * REL_L2, what


def _tiny():
    return si.Decoder("tiny-glue", layers=2, hidden=512, q_heads=4, mlp=1280, vocab=1000,
                      kv_heads=2, head_dim=64)


def _glue_stack(qd, fmt, m, d):
    """A decode step whose projections feed each other through the glue:
    RMSNorm before q|k|v, gate|up and the head; silu on gate; the gated
    product before down; each layer's input is the previous down's output.
    The attention output feeding o is a synthetic activation (attention is
    outside the linear path).  Returns the device ops and, per op, what the
    oracle needs to recompute it."""
    H, Q, I = d.hidden, d.q_dim, d.mlp
    shape = (lambda n: (m, n) if m > 1 else (n,))
    nan = lambda n: torch.full(shape(n), float("nan"), dtype=torch.float16, device=DEV)
    x_in = _gpu(si.activations(si.seed_for("gs-x0", m), m, H).reshape(shape(H)))
    ops, meta, gid = [], [], 0
    keep = []
    for layer in range(d.layers):
        g_attn = _gpu(si.norm_weight(si.seed_for("gs-ga", layer), H))
        g_mlp = _gpu(si.norm_weight(si.seed_for("gs-gm", layer), H))
        keep += [g_attn, g_mlp]
        for pname, n in ((f"L{layer}.q", Q), (f"L{layer}.k", d.kv_dim), (f"L{layer}.v", d.kv_dim)):
            w = si.weights(si.seed_for("gs-w", pname), n, H)
            op = qd.LinearOp(_pack(qd, fmt, w), x_in, nan(n), gid, prologue="rmsnorm", gamma=g_attn,
                             eps=EPS)
            ops.append(op)
            meta.append((pname, w, "rmsnorm", g_attn, "none"))
        gid += 1
        attn = _gpu(si.activations(si.seed_for("gs-attn", layer, m), m, Q).reshape(shape(Q)))
        keep.append(attn)
        w = si.weights(si.seed_for("gs-w", f"L{layer}.o"), H, Q)
        o_y = nan(H)
        ops.append(qd.LinearOp(_pack(qd, fmt, w), attn, o_y, gid))
        meta.append((f"L{layer}.o", w, "none", None, "none"))
        gid += 1
        gu = torch.full((2 * m * I,), float("nan"), dtype=torch.float16, device=DEV)
        keep.append(gu)
        for j, (pname, epi) in enumerate(((f"L{layer}.gate", "silu"), (f"L{layer}.up", "none"))):
            w = si.weights(si.seed_for("gs-w", pname), I, H)
            y = gu[j * m * I:(j + 1) * m * I].view(shape(I))
            ops.append(qd.LinearOp(_pack(qd, fmt, w), o_y, y, gid, prologue="rmsnorm", gamma=g_mlp,
                                   eps=EPS, epilogue=epi))
            meta.append((pname, w, "rmsnorm", g_mlp, epi))
        gid += 1
        w = si.weights(si.seed_for("gs-w", f"L{layer}.down"), H, I)
        down_y = nan(H)
        ops.append(qd.LinearOp(_pack(qd, fmt, w), gu, down_y, gid, prologue="glu"))
        meta.append((f"L{layer}.down", w, "glu", None, "none"))
        gid += 1
        x_in = down_y
    g_fin = _gpu(si.norm_weight(si.seed_for("gs-gf"), H))
    keep.append(g_fin)
    w = si.weights(si.seed_for("gs-w", "head"), d.vocab, H)
    ops.append(qd.LinearOp(_pack(qd, fmt, w), x_in, nan(d.vocab), gid, prologue="rmsnorm",
                           gamma=g_fin, eps=EPS))
    meta.append(("head", w, "rmsnorm", g_fin, "none"))
    return ops, meta, keep


def _check_glue_stack(fmt, m, ops, meta, tag):
    for op, (pname, w, pro, gam, epi) in zip(ops, meta):
        x_dev = _host(op.x).astype(np.float16)
        k = w.shape[1]
        if pro == "glu":
            xin = glue.apply_prologue("glu", x_dev.reshape(2, m, k))
        elif pro == "rmsnorm":
            xin = glue.rmsnorm_fp16(x_dev.reshape(m, k), _host(gam), EPS)
        else:
            xin = x_dev.reshape(m, k)
        assert np.all(np.isfinite(xin.astype(np.float64))), f"{tag} {pname}: non-finite input"
        parts = _parts(fmt, w)
        ref = linear.ref_linear(fmt, parts, xin).reshape(m, -1)
        rmax = linear.row_max_abs(fmt, parts)
        y = _host(op.y).reshape(m, -1)
        for t in range(m):
            if epi == "silu":
                _check_silu(y[t], ref[t], rmax, xin[t], f"{tag} {pname} token {t}")
            else:
                check_vector(y[t], ref[t], rmax, xin[t], f"{tag} {pname} token {t}")


@pytest.mark.parametrize("fmt,m", [("int8_b32", 1), ("int4_g64", 1), ("fp16", 1), ("int8_b32", 16),
                                   ("int4_g64", 16), ("fp16", 5)])
def test_glue_stack_launches(qd, fmt, m):
    ops, meta, keep = _glue_stack(qd, fmt, m, _tiny())
    qd.decode_linear_stack(ops, m)
    _check_glue_stack(fmt, m, ops, meta, f"launches {fmt} m={m}")


@pytest.mark.parametrize("fmt,m", [("int8_b32", 16), ("int4_g64", 16), ("int8_b32", 5), ("int4_g64", 2),
                                   ("fp16", 5)])
def test_glue_stack_plan_multi_token(qd, fmt, m):
    """A plan of the glued step at m > 1: the persistent kernel runs all of
    it (int8, INT4; fp16 replays launches).  Each op against the oracle on
    the activations it read, and bit-identical repeated runs with the outputs
    poisoned in between: the RMSNorm factors come from per-workgroup records
    added in a fixed order, gate|up runs paired and writes down's gated
    product."""
    ops, meta, keep = _glue_stack(qd, fmt, m, _tiny())
    plan = qd.StackPlan(ops, m)
    assert plan.persistent == (fmt != "fp16")
    if fmt != "fp16":
        d = qd.describe_stack_plan(ops, m)
        assert d[4] == 1 and d[5] == len(ops), "the whole glued step runs in the persistent kernel"
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
            _check_glue_stack(fmt, m, ops, meta, f"plan {fmt} m={m}")
        else:
            for a, b in zip(first, outs):
                assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    plan.close()


@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
def test_glue_stack_plan_parity_and_determinism(qd, fmt):
    """A plan of the glued step (the persistent kernel at one token row): per-op
    parity and bit-identical repeated runs, outputs poisoned in between."""
    ops, meta, keep = _glue_stack(qd, fmt, 1, _tiny())
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
            _check_glue_stack(fmt, 1, ops, meta, f"plan {fmt}")
        else:
            for a, b in zip(first, outs):
                assert np.array_equal(a.view(np.uint16), b.view(np.uint16))
    plan.close()


@pytest.mark.parametrize("fmt", ["int8_b32", "int4_g64"])
def test_glue_stack_persistent(qd, fmt):
    """The glued step in the one-launch persistent kernel (staging applies the
    prologue in LDS, after x's whole LDS span, so K not a multiple of 512
    stays inside the region): per-op parity."""
    ops, meta, keep = _glue_stack(qd, fmt, 1, _tiny())
    plan = qd.StackPlan(ops, 1)
    assert plan.persistent
    plan.run()
    torch.cuda.synchronize()
    assert plan.error() == 0
    _check_glue_stack(fmt, 1, ops, meta, f"persistent {fmt}")
    plan.close()


@pytest.mark.parametrize("workload,path", [("qwen3-8b-int8-glue-m1", "launches"),
                                           ("qwen3-8b-int8-glue-m1", "plan"),
                                           ("qwen3-8b-int8-glue-m16", "launches"),
                                           ("qwen3-8b-int8-glue-m16", "plan")])
def test_glue_full_size_sampled(qd, workload, path):
    """The full 8B-shaped step chained through the glue, as the bench times it
    (the persistent plan, per-group launches): every output
    finite; sampled rows of sampled projections (RMSNorm-fed q and head,
    silu-stored gate, up, gated-product-fed down, plain o) match the oracle on
    the activations each op read."""
    import bench
    ops, alg_bytes, weight_bytes, m = bench.build_stack(qd, si, torch, workload, DEV)
    for op in ops:
        op.y.fill_(float("nan"))
    if path == "plan":
        plan = qd.StackPlan(ops, m)
        assert plan.persistent
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        plan.close()
    else:
        qd.decode_linear_stack(ops, m)
    torch.cuda.synchronize()
    wl = si.WORKLOADS[workload]
    d = wl.decoder
    names = [p for _, ms in d.groups() for p, _, _ in ms]
    assert len(names) == len(ops)
    for op in ops:
        assert torch.isfinite(op.y).all()
    last, mid = d.layers - 1, d.layers // 2
    rng = np.random.default_rng(14)
    for name in ["L0.q", f"L{mid}.gate", f"L{mid}.up", f"L{last}.down", f"L{last}.o", "head"]:
        op = ops[names.index(name)]
        n, k = op.w.n, op.w.k
        x_dev = _host(op.x).astype(np.float16)
        if op.prologue == "glu":
            xin = glue.apply_prologue("glu", x_dev.reshape(2, m, k))
        elif op.prologue == "rmsnorm":
            xin = glue.rmsnorm_fp16(x_dev.reshape(m, k), _host(op.gamma), op.eps)
        else:
            xin = x_dev.reshape(m, k)
        rows = np.sort(rng.choice(n, 16, replace=False))
        w_rows = si.weights_torch(si.matrix_seed(d.name, name), n, k, DEV)[rows].cpu().numpy()
        parts = _parts(wl.fmt, w_rows)
        ref = linear.ref_linear(wl.fmt, parts, xin).reshape(m, -1)
        rmax = linear.row_max_abs(wl.fmt, parts)
        y = _host(op.y).reshape(m, -1)[:, rows]
        for t in range(m):
            if op.epilogue == "silu":
                _check_silu(y[t], ref[t], rmax, xin[t], f"{name} token {t}")
            else:
                check_vector(y[t], ref[t], rmax, xin[t], f"{name} token {t}")
    del ops
    torch.cuda.empty_cache()


def test_plan_random_glued_steps_against_sequential_model(qd):
    """Random one-token steps with glue, run by the persistent kernel's glued
    instance, against a sequential model of the buffers built from the
    oracle: each group takes no prologue, RMSNorm (its own gamma) or the
    gated product of two blocks, and each member stores with or without
    silu.  Inputs are fresh, an earlier op's output or a slice of one;
    outputs are fresh or overwrite an earlier output.  Every group is checked
    on the input the device gave it, at the acceptance bound."""
    from int4_quantized_decode_amd import LinearOp
    rng = np.random.default_rng(si.seed_for("random-glued-steps"))
    arena_n = 1 << 20
    for case in range(16):
        fmt = ["int8_b32", "int4_g64"][case % 2]
        init = si.activations(si.seed_for("random-glued-arena", case), 1, arena_n)[0]
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
            pro = ["none", "rmsnorm", "glu"][int(rng.integers(3))]
            span = 2 * k if pro == "glu" else k
            cands = [(o, n) for o, n in outs if n >= span]
            if cands and rng.random() < 0.6:
                o, n = cands[int(rng.integers(len(cands)))]
                xo = o + 8 * int(rng.integers(0, (n - span) // 8 + 1))
            else:
                xo = take(span)
            gamma = None
            if pro == "rmsnorm":
                gamma = _gpu((1.0 + 0.25 * rng.standard_normal(k)).astype(np.float16))
            members = []
            for _ in range(int(rng.integers(1, 4))):
                n = int(rng.choice([16, 48, 100, 256, 1000, 2176]))
                same = [o for o, nn in outs if nn == n and not (o < xo + span and xo < o + n)
                        and all(o != mo for mo, _, _, _ in members)]
                yo = same[0] if same and rng.random() < 0.25 else take(n)
                epi = "silu" if rng.random() < 0.4 else "none"
                w = si.weights(si.seed_for("random-glued-w", case, g, len(members)), n, k)
                members.append((yo, n, w, epi))
            for yo, n, w, epi in members:
                ops.append(LinearOp(_pack(qd, fmt, w), arena[xo:xo + span], arena[yo:yo + n], g,
                                    prologue=pro, gamma=gamma, eps=EPS if pro == "rmsnorm" else 0.0,
                                    epilogue=epi))
            prog.append((xo, k, span, pro, None if gamma is None else _host(gamma), members))
            outs.extend((yo, n) for yo, n, _, _ in members)
        plan = qd.StackPlan(ops, 1)
        assert plan.persistent, f"case {case}"
        init_g = _gpu(init)

        def restore():
            arena.copy_(init_g)

        def snapshot():
            return _host(arena).copy()

        # Plans of the step's first groups give the arena after each group:
        # every output against the oracle's glue and product on the raw
        # input the device gave the group, at the acceptance bound (silu
        # outputs: that bound through silu), nothing else changed; then the
        # one-plan step must reproduce the final arena bit for bit.
        states = _prefix_states(qd, ops, 1, restore, snapshot)
        for g, (xo, k, span, pro, gam, members) in enumerate(prog):
            raw = states[g][xo:xo + span]
            assert np.all(np.isfinite(raw.astype(np.float64))), f"case {case} group {g} input"
            X = glue.apply_prologue(pro, raw, gam, EPS).astype(np.float64)
            touched = np.zeros(arena_n, bool)
            for yo, n, w, epi in members:
                parts = _parts(fmt, w)
                Y = linear.ref_linear(fmt, parts, X)
                got = states[g + 1][yo:yo + n]
                rmax = linear.row_max_abs(fmt, parts)
                if epi == "silu":
                    _check_silu(got, Y, rmax, X, f"case {case} ({fmt}) group {g} silu output at {yo}")
                else:
                    check_vector(got, Y, rmax, X, f"case {case} ({fmt}) group {g} output at {yo}")
                touched[yo:yo + n] = True
            assert np.array_equal(states[g + 1][~touched].view(np.uint16), states[g][~touched].view(np.uint16)), \
                f"case {case} group {g} wrote outside its outputs"
        restore()
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        assert np.array_equal(snapshot().view(np.uint16), states[-1].view(np.uint16)), f"case {case}"
        plan.close()


def test_plan_random_glued_steps_multi_token(qd):
    """Random glued steps at 2, 5 and 16 token rows against a sequential
    model of the buffers built from the oracle.  Groups take no prologue,
    RMSNorm or the gated product; inputs are fresh, an earlier op's whole
    output (so RMSNorm's factors come from the producing op's per-workgroup
    records) or the two outputs of an earlier two-op group written one after
    the other (so that group runs paired and writes the product); ops store
    with or without silu.  Where a glued group falls outside what the
    persistent kernel takes, the rest of the step replays launches.  Every
    group is checked on the input the device gave it, at the acceptance
    bound, nothing else may change, and the one-plan step must reproduce the
    final buffers bit for bit."""
    from int4_quantized_decode_amd import LinearOp
    rng = np.random.default_rng(si.seed_for("random-glued-steps-multi"))
    arena_n = 1 << 21
    seen_paired = seen_records = 0
    for case in range(12):
        fmt = ["int8_b32", "int4_g64"][case % 2]
        m = [2, 5, 16][case % 3]
        init = si.activations(si.seed_for("random-glued-arena-multi", case), 1, arena_n)[0]
        arena = _gpu(init)
        top = 0

        def take(n):
            nonlocal top
            off = top
            top += (n + 63) // 64 * 64
            assert top <= arena_n
            return off

        ops, prog, outs, pairs = [], [], [], []
        for g in range(int(rng.integers(2, 7))):
            pro = ["none", "rmsnorm", "glu"][int(rng.integers(3))]
            k = int(rng.choice([256, 512, 1088]))
            if pro == "glu" and pairs and rng.random() < 0.7:
                xo, k = pairs[int(rng.integers(len(pairs)))]
            elif pro != "glu" and any(n % 64 == 0 for _, n in outs) and rng.random() < 0.6:
                cands = [(o, n) for o, n in outs if n % 64 == 0]      # a K both formats take
                xo, k = cands[int(rng.integers(len(cands)))]
            else:
                xo = take(m * k * (2 if pro == "glu" else 1))
            span = m * k * (2 if pro == "glu" else 1)
            gamma = None
            if pro == "rmsnorm":
                gamma = _gpu((1.0 + 0.25 * rng.standard_normal(k)).astype(np.float16))
            members = []
            if rng.random() < 0.4:
                n = int(rng.choice([256, 512, 1088]))
                go = take(2 * m * n)
                for j in range(2):
                    epi = "silu" if (j == 0 and rng.random() < 0.7) else "none"
                    w = si.weights(si.seed_for("random-glued-multi-w", case, g, j), n, k)
                    members.append((go + j * m * n, n, w, epi))
                pairs.append((go, n))
            else:
                for j in range(int(rng.integers(1, 4))):
                    n = int(rng.choice([16, 48, 256, 1000, 1088]))
                    epi = "silu" if rng.random() < 0.4 else "none"
                    w = si.weights(si.seed_for("random-glued-multi-w", case, g, j), n, k)
                    members.append((take(m * n), n, w, epi))
            for yo, n, w, epi in members:
                ops.append(LinearOp(_pack(qd, fmt, w), arena[xo:xo + span].view(-1, k) if pro != "glu"
                                    else arena[xo:xo + span], arena[yo:yo + m * n].view(m, n), g,
                                    prologue=pro, gamma=gamma, eps=EPS if pro == "rmsnorm" else 0.0,
                                    epilogue=epi))
            prog.append((xo, k, span, pro, None if gamma is None else _host(gamma), members))
            outs.extend((yo, n) for yo, n, _, _ in members)
        v, groups, _, _ = _plan_tables(qd, ops, m)
        assert v[1] == 1, f"case {case}"
        seen_paired += any(g[8] & 16 for g in groups)          # a paired group writes a gated product
        seen_records += v[16] > 0                               # sum-of-squares records
        init_g = _gpu(init)

        def restore():
            arena.copy_(init_g)

        def snapshot():
            return _host(arena).copy()

        states = _prefix_states(qd, ops, m, restore, snapshot)
        for g, (xo, k, span, pro, gam, members) in enumerate(prog):
            raw = states[g][xo:xo + span]
            assert np.all(np.isfinite(raw.astype(np.float64))), f"case {case} group {g} input"
            raw = raw.reshape(2, m, k) if pro == "glu" else raw.reshape(m, k)
            X = glue.apply_prologue(pro, raw, gam, EPS).astype(np.float64)
            touched = np.zeros(arena_n, bool)
            for yo, n, w, epi in members:
                parts = _parts(fmt, w)
                Y = linear.ref_linear(fmt, parts, X)
                got = states[g + 1][yo:yo + m * n].reshape(m, n)
                rmax = linear.row_max_abs(fmt, parts)
                for t in range(m):
                    what = f"case {case} ({fmt}, m={m}) group {g} {pro} output at {yo} token {t}"
                    if epi == "silu":
                        _check_silu(got[t], Y[t], rmax, X[t], what)
                    else:
                        check_vector(got[t], Y[t], rmax, X[t], what)
                touched[yo:yo + m * n] = True
            assert np.array_equal(states[g + 1][~touched].view(np.uint16), states[g][~touched].view(np.uint16)), \
                f"case {case} group {g} wrote outside its outputs"
        plan = qd.StackPlan(ops, m)
        restore()
        plan.run()
        torch.cuda.synchronize()
        assert plan.error() == 0
        assert np.array_equal(snapshot().view(np.uint16), states[-1].view(np.uint16)), f"case {case}"
        plan.close()
    assert seen_paired >= 2 and seen_records >= 2
