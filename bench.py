#!/usr/bin/env python3
"""Benchmark one decode step's quantized linear stack on one MI355X.

A step is one pass over every projection of a Qwen3-8B-shaped decoder (36
layers x [q|k|v] -> o -> [gate|up] -> down, then the 151 936-row head) with
int8 b32 weights and one fp16 activation vector per group, all resident in HBM
before timing starts.  The metric is the algorithmic bytes a step must move
(packed weights + activations + outputs) divided by the time per step.

Prints one JSON line.  Run with no flags for the default workload.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

HBM_PEAK_GBS = 8000.0            # MI355X HBM3E, 8 TB/s
METRIC = "achieved HBM GB/s and us per decode step (8B-shaped int8 b32 stack, M=1)"


def parse():
    ap = argparse.ArgumentParser(description=__doc__)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--workload", default="qwen3-8b-int8-m1")
    ap.add_argument("--path", choices=["plan", "launches"], default="plan",
                    help="plan: persistent one-launch step (default); launches: one fused launch per group")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-chain", action="store_true",
                    help="default workload only: skip the chained step measured beside it")
    ap.add_argument("--rotate-mb", type=int, default=1024,
                    help="single-GEMV workload: weight copies cycled to exceed the caches")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only copy 1 GiB device to device (reference kernel for HBM counters)")
    return ap.parse_args()


def log(msg):
    print(f"[bench] {msg}", file=sys.stderr, flush=True)


def build_stack(qd, si, torch, workload, dev):
    wl = si.WORKLOADS[workload]
    m = wl.m
    if wl.glue:
        return build_glue_stack(qd, si, torch, workload, dev)
    if wl.chain:
        return build_chain_stack(qd, si, torch, workload, dev)
    if wl.single is not None:
        n, k = wl.single
        groups, model = [("gemv", [("W", n, k)])], "single"
    else:
        groups, model = wl.decoder.groups(), wl.decoder.name
    ops, alg_bytes, weight_bytes = [], 0, 0
    for gi, (gname, members) in enumerate(groups):
        k = members[0][2]
        x = si.activations(si.activation_seed(workload, gname), m, k)
        x_gpu = torch.from_numpy(x if m > 1 else x[0]).to(dev)
        alg_bytes += m * k * 2
        for pname, n, kk in members:
            w = si.weights_torch(si.matrix_seed(model, pname), n, kk, dev)
            fmt = wl.head_fmt if (pname == "head" and wl.head_fmt) else wl.fmt
            pw = PACKERS[fmt](qd)(w)
            del w
            y = torch.empty((m, n) if m > 1 else (n,), dtype=torch.float16, device=dev)
            ops.append(qd.LinearOp(pw, x_gpu, y, gi))
            alg_bytes += pw.blob.numel() + m * n * 2
            weight_bytes += pw.blob.numel()
    torch.cuda.synchronize()
    return ops, alg_bytes, weight_bytes, m


PACKERS = {"int8_b32": lambda qd: qd.qpack_int8_b32, "int4_g64": lambda qd: qd.qpack_int4_g64,
           "fp16": lambda qd: qd.qpack_fp16}
GLUE_EPS = 1e-6


def build_chain_stack(qd, si, torch, workload, dev):
    """The decoder step with a true dependency at every boundary (each group
    reads an earlier group's output; see synthetic_inputs).  Weights are
    drawn as for the other workloads and scaled to standard deviation
    1/sqrt(K), so that activations keep their size along the 145-group
    chain instead of overflowing fp16; quantized bytes and timing do not
    depend on that scale."""
    wl = si.WORKLOADS[workload]
    m, d = wl.m, wl.decoder
    H, Q, I = d.hidden, d.q_dim, d.mlp
    shape = (lambda n: (m, n) if m > 1 else (n,))
    ops, alg_bytes, weight_bytes = [], 0, 0
    gi = 0

    def add(pname, n, k, x, fmt=wl.fmt):
        nonlocal alg_bytes, weight_bytes
        w = si.weights_torch(si.matrix_seed(d.name, pname), n, k, dev)
        w.mul_(1.0 / (si.W_STD * k ** 0.5))
        pw = PACKERS[fmt](qd)(w)
        del w
        y = torch.empty(shape(n), dtype=torch.float16, device=dev)
        ops.append(qd.LinearOp(pw, x, y, gi))
        alg_bytes += pw.blob.numel() + m * n * 2
        weight_bytes += pw.blob.numel()
        return y

    x_in = torch.from_numpy(si.activations(si.activation_seed(workload, "x0"), m, H)
                            .reshape(shape(H))).to(dev)
    for layer in range(d.layers):
        alg_bytes += m * H * 2
        q_y = add(f"L{layer}.q", Q, H, x_in)
        add(f"L{layer}.k", d.kv_dim, H, x_in)
        add(f"L{layer}.v", d.kv_dim, H, x_in)
        gi += 1
        alg_bytes += m * Q * 2
        o_y = add(f"L{layer}.o", H, Q, q_y)
        gi += 1
        alg_bytes += m * H * 2
        gate_y = add(f"L{layer}.gate", I, H, o_y)
        add(f"L{layer}.up", I, H, o_y)
        gi += 1
        alg_bytes += m * I * 2
        x_in = add(f"L{layer}.down", H, I, gate_y)
        gi += 1
    alg_bytes += m * H * 2
    add("head", d.vocab, H, x_in, fmt=wl.head_fmt or wl.fmt)
    torch.cuda.synchronize()
    return ops, alg_bytes, weight_bytes, m


def build_glue_stack(qd, si, torch, workload, dev):
    """The decoder step chained through the fused glue: each layer's q|k|v
    and gate|up read the RMSNorm of their input (the previous layer's down
    output, the o output), gate stores silu, down reads the gated product of
    the gate and up outputs, the head reads the RMSNorm of the last down
    output.  o reads a synthetic attention output.  Algorithmic bytes add
    the norm weights and down's second input block."""
    wl = si.WORKLOADS[workload]
    m, d = wl.m, wl.decoder
    H, Q, I = d.hidden, d.q_dim, d.mlp
    shape = (lambda n: (m, n) if m > 1 else (n,))
    fmt = wl.fmt
    ops, alg_bytes, weight_bytes = [], 0, 0
    gi = 0

    def add(pname, n, k, x, y, **glue):
        nonlocal alg_bytes, weight_bytes
        w = si.weights_torch(si.matrix_seed(d.name, pname), n, k, dev)
        pw = PACKERS[fmt](qd)(w)
        del w
        ops.append(qd.LinearOp(pw, x, y, gi, **glue))
        alg_bytes += pw.blob.numel() + m * n * 2
        weight_bytes += pw.blob.numel()

    def norm_w(*tag):
        return torch.from_numpy(si.norm_weight(si.seed_for("gamma", d.name, *tag), H)).to(dev)

    x_in = torch.from_numpy(si.activations(si.activation_seed(workload, "x0"), m, H)
                            .reshape(shape(H))).to(dev)
    for layer in range(d.layers):
        g_attn, g_mlp = norm_w("attn", layer), norm_w("mlp", layer)
        alg_bytes += m * H * 2 + H * 2
        for pname, n in ((f"L{layer}.q", Q), (f"L{layer}.k", d.kv_dim), (f"L{layer}.v", d.kv_dim)):
            add(pname, n, H, x_in, torch.empty(shape(n), dtype=torch.float16, device=dev),
                prologue="rmsnorm", gamma=g_attn, eps=GLUE_EPS)
        gi += 1
        attn = torch.from_numpy(si.activations(si.activation_seed(workload, f"L{layer}.attn"), m, Q)
                                .reshape(shape(Q))).to(dev)
        o_y = torch.empty(shape(H), dtype=torch.float16, device=dev)
        alg_bytes += m * Q * 2
        add(f"L{layer}.o", H, Q, attn, o_y)
        gi += 1
        gu = torch.empty(2 * m * I, dtype=torch.float16, device=dev)
        alg_bytes += m * H * 2 + H * 2
        add(f"L{layer}.gate", I, H, o_y, gu[:m * I].view(shape(I)), prologue="rmsnorm", gamma=g_mlp,
            eps=GLUE_EPS, epilogue="silu")
        add(f"L{layer}.up", I, H, o_y, gu[m * I:].view(shape(I)), prologue="rmsnorm", gamma=g_mlp,
            eps=GLUE_EPS)
        gi += 1
        x_in = torch.empty(shape(H), dtype=torch.float16, device=dev)
        alg_bytes += 2 * m * I * 2
        add(f"L{layer}.down", H, I, gu, x_in, prologue="glu")
        gi += 1
    g_fin = norm_w("final")
    alg_bytes += m * H * 2 + H * 2
    head_fmt = wl.head_fmt or fmt
    w = si.weights_torch(si.matrix_seed(d.name, "head"), d.vocab, H, dev)
    pw = PACKERS[head_fmt](qd)(w)
    del w
    ops.append(qd.LinearOp(pw, x_in, torch.empty(shape(d.vocab), dtype=torch.float16, device=dev), gi,
                           prologue="rmsnorm", gamma=g_fin, eps=GLUE_EPS))
    alg_bytes += pw.blob.numel() + m * d.vocab * 2
    weight_bytes += pw.blob.numel()
    torch.cuda.synchronize()
    return ops, alg_bytes, weight_bytes, m


def recorded_traffic(kernel_tag, workload):
    """HBM bytes per launch of the timed kernel as last measured with
    rocprofv3 counters (FETCH_SIZE and WRITE_SIZE, each scaled by the same
    counter's reading for a plain copy of known size), from the committed
    summary under profiles/.  None when there is no summary, or when the
    kernel's source has changed since the counters were taken (the summary
    records a hash of the sources)."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"traffic_{kernel_tag}_{workload}.txt")
    if not os.path.exists(path):
        return None
    fields = {}
    for line in open(path):
        if ":" in line and not line.startswith(" "):
            key, _, val = line.partition(":")
            fields[key.strip()] = val.strip()
    srcs = fields.get("sources", "").split()
    h = hashlib.sha256()
    for rel in srcs:
        with open(os.path.join(ROOT, rel), "rb") as f:
            h.update(f.read())
    if not srcs or h.hexdigest()[:16] != fields.get("sources_sha256_16"):
        return None
    try:
        return int(fields["hbm_bytes_per_launch"])
    except (KeyError, ValueError):
        return None


def read_probe_gbs(qd, torch, dev, gib=2, reps=7):
    """Best-of-grid median bandwidth of a plain streaming read of `gib` GiB
    (the library's read probe), measured in this run."""
    buf = torch.empty(gib << 30, dtype=torch.uint8, device=dev)
    sink = torch.zeros(1, dtype=torch.int32, device=dev)
    best = 0.0
    for grid in (256, 512, 1024):
        qd.read_probe(buf, sink, grid)                 # warm
        evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
               for _ in range(reps)]
        for a, b in evs:
            a.record()
            qd.read_probe(buf, sink, grid)
            b.record()
        torch.cuda.synchronize()
        ms = sorted(a.elapsed_time(b) for a, b in evs)[reps // 2]
        best = max(best, buf.numel() / (ms * 1e-3) / 1e9)
    del buf
    torch.cuda.empty_cache()
    return best


def _cpu_model() -> str:
    try:
        for line in open("/proc/cpuinfo"):
            if line.startswith("model name"):
                return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def _synthetic_parts(rng, fmt, n, k):
    """Canonical quantized arrays of one [n, k] matrix with the format's
    shapes and value ranges, drawn directly (timing only: the oracle's cost
    does not depend on the values, and quantizing gigabytes on the host is
    slower than the products being timed)."""
    import numpy as np
    if fmt == "int8_b32":
        return (rng.integers(-127, 128, (n, k), dtype=np.int8),
                (rng.standard_normal((n, k // 32)) * 2e-4).astype(np.float16))
    return (rng.integers(0, 16, (n, k), dtype=np.uint8),
            (rng.standard_normal((n, k // 64)) * 1e-3).astype(np.float16),
            (rng.standard_normal((n, k // 64)) * 2e-2).astype(np.float16))


def cpu_baseline(si, workload, alg_bytes_step):
    """The oracle as it stands (fp64 dequantize-then-multiply, matrices
    streamed in row chunks), timed on this host over every projection of one
    full step of the workload, with BLAS threads pinned to the cores this
    process may run on.  Codes and scales are drawn once per distinct matrix
    shape and reused across layers."""
    import numpy as np
    from oracle import linear
    cores = len(os.sched_getaffinity(0))
    try:
        from threadpoolctl import threadpool_limits
        limiter = threadpool_limits(cores)
    except Exception:
        limiter = None
    wl = si.WORKLOADS[workload]
    if wl.single is not None:
        n, k = wl.single
        groups, model = [("gemv", [("W", n, k)])], "single"
    else:
        groups, model = wl.decoder.groups(), wl.decoder.name
    rng = np.random.default_rng(20261203)
    parts_by_shape, xs = {}, {}
    for gname, members in groups:
        k = members[0][2]
        if k not in xs:
            x = si.activations(si.activation_seed(workload, "cpu", k), wl.m, k)
            xs[k] = x if wl.m > 1 else x[0]
        for pname, n, kk in members:
            if (n, kk) not in parts_by_shape:
                parts_by_shape[(n, kk)] = _synthetic_parts(rng, wl.fmt, n, kk)
    t0 = time.perf_counter()
    for gname, members in groups:
        for pname, n, kk in members:
            linear.ref_linear(wl.fmt, parts_by_shape[(n, kk)], xs[kk])
    secs = time.perf_counter() - t0
    if limiter is not None:
        limiter.unregister()
    return {"value": round(alg_bytes_step / secs / 1e9, 3), "unit": "GB/s", "cores": cores, "kind": "oracle",
            "us_per_step": round(secs * 1e6, 1), "cpu_model": _cpu_model(),
            "sample": f"one full step of {workload} ({sum(len(m) for _, m in groups)} projections, every one "
                      f"computed once), fp64 dequantize-then-multiply in row chunks of {linear.ROW_CHUNK}, "
                      f"{secs:.1f} s; codes and scales drawn per matrix shape, not quantized from the step's weights"}


TRIALS = 3

# The pages' whole-model decode rates on an Apple M4 Max (int8hu bundles):
# Qwen3-VL 4B and 8B Core AI cards, Measured paragraph; Qwen3.8-27B page,
# Verified table (llm-benchmark -n 3).  Context only: another machine, and a
# whole decoder rather than its linear layers.
M4_MAX_DECODE_TOK_S = {"qwen3-vl-4b": 92.2, "qwen3-vl-8b": 54.3, "qwen3.8-27b": 15.7}


def time_steps(run, steps, stream, torch):
    """`steps` steps bracketed by a synchronize on both sides; HIP events on
    the launch stream around each step.  Returns (wall seconds per step,
    per-step event milliseconds)."""
    evs = [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)) for _ in range(steps)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i, (a, b) in enumerate(evs):
        a.record(stream)
        run(i)
        b.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) / steps
    return wall, [a.elapsed_time(b) for a, b in evs]


def measure(qd, si, torch, workload, path, steps, warmup, rotate_mb, dev):
    """Build a workload, warm up, then TRIALS timed trials of `steps` steps."""
    log(f"building {workload} (weights generated and packed on the device)")
    ops, alg_bytes, weight_bytes, m = build_stack(qd, si, torch, workload, dev)
    log(f"{len(ops)} projections, {weight_bytes / 1e9:.3f} GB packed weights, {alg_bytes / 1e9:.4f} GB per step")
    wl = si.WORKLOADS[workload]
    per_step = 1
    if wl.single is not None:
        # One step is a pass over copies of the one matrix (so that no copy is
        # still in the caches when it is read again), each GEMV its own group
        # with its own output, issued by one library call: the GEMVs run back
        # to back with no host work between them (launches: one per GEMV;
        # plan: one persistent launch, the GEMVs independent of each other).
        copies = max(1, (rotate_mb << 20) // max(1, weight_bytes))
        op = ops[0]
        step_ops = [[op] + [qd.LinearOp(qd.PackedWeight(op.w.fmt, op.w.n, op.w.k, op.w.blob.clone()),
                                        op.x, torch.empty_like(op.y), i + 1) for i in range(copies - 1)]]
        per_step = copies
        alg_bytes *= copies
        weight_bytes *= copies
    else:
        step_ops = [ops]
    plans = []
    if path == "plan":
        plans = [qd.StackPlan(o, m) for o in step_ops]
        runners = [p.run for p in plans]
    else:
        runners = [(lambda o=o: qd.decode_linear_stack(o, m)) for o in step_ops]
    stream = torch.cuda.current_stream()
    run = lambda i: runners[i % len(runners)]()  # noqa: E731
    for i in range(warmup):
        run(i)
    torch.cuda.synchronize()
    trials = []
    for t in range(TRIALS):
        wall, ev_ms = time_steps(run, steps, stream, torch)
        trials.append((wall, ev_ms))
        log(f"{workload} trial {t}: wall {wall * 1e6:.1f} us/step, event median "
            f"{sorted(ev_ms)[len(ev_ms) // 2] * 1e3:.1f} us")
    for p in plans:
        if p.error():
            raise RuntimeError("stack plan reported a timed-out wait")
    persistent = path == "plan" and all(p.persistent for p in plans)
    ngroups = len({op.group for op in step_ops[0]})
    for p in plans:
        p.close()
    return {"ops": ops, "n_ops": len(step_ops[0]), "alg_bytes": alg_bytes, "weight_bytes": weight_bytes, "m": m,
            "wl": wl, "trials": trials, "persistent": persistent, "ngroups": ngroups, "per_step": per_step}


def summarize(res):
    walls = sorted(w for w, _ in res["trials"])
    med_wall = walls[len(walls) // 2]
    all_ev = sorted(e for _, ev in res["trials"] for e in ev)
    return {"wall_s": med_wall, "trials_us": [round(w * 1e6, 2) for w, _ in res["trials"]],
            "spread_us": round((walls[-1] - walls[0]) * 1e6, 2),
            "ev_mean_s": sum(all_ev) / len(all_ev) * 1e-3,
            "ev_p10_us": all_ev[len(all_ev) // 10] * 1e3, "ev_p50_us": all_ev[len(all_ev) // 2] * 1e3,
            "ev_p90_us": all_ev[(9 * len(all_ev)) // 10] * 1e3}


def main():
    args = parse()
    if args.copy_calibration:
        import torch
        src = torch.ones(1 << 30, dtype=torch.uint8, device="cuda:0")
        dst = torch.empty_like(src)
        torch.cuda.synchronize()
        dst.copy_(src)
        torch.cuda.synchronize()
        print(json.dumps({"copy_bytes": 1 << 30}))
        return
    if args.gpus != 1:
        print(json.dumps({"error": "this build runs on one GPU only; --gpus must be 1"}))
        sys.exit(2)
    import torch
    import int4_quantized_decode_amd as qd
    import synthetic_inputs as si

    dev = "cuda:0"
    torch.cuda.set_device(0)
    res = measure(qd, si, torch, args.workload, args.path, args.steps, args.warmup, args.rotate_mb, dev)
    sm = summarize(res)
    alg_bytes, m, wl = res["alg_bytes"], res["m"], res["wl"]
    wall_ms = sm["wall_s"] * 1e3
    value = alg_bytes / sm["wall_s"] / 1e9
    log(f"wall {wall_ms * 1e3:.1f} us/step (median of {TRIALS} trials {sm['trials_us']}), event median "
        f"{sm['ev_p50_us']:.1f} us (p10 {sm['ev_p10_us']:.1f}, p90 {sm['ev_p90_us']:.1f})")

    chained = None
    if args.workload == "qwen3-8b-int8-m1" and args.path == "plan" and not args.no_chain:
        # The same step with a true dependency at every boundary (each group
        # reads an earlier group's output): the decode a real model runs.
        del res["ops"]
        torch.cuda.empty_cache()
        cres = measure(qd, si, torch, "qwen3-8b-int8-chain-m1", "plan", args.steps, args.warmup, 0, dev)
        csm = summarize(cres)
        chained = {"workload": "qwen3-8b-int8-chain-m1", "us_per_step": round(csm["wall_s"] * 1e6, 2),
                   "trials_us": csm["trials_us"], "spread_us": csm["spread_us"],
                   "gbs": round(cres["alg_bytes"] / csm["wall_s"] / 1e9, 2),
                   "frac_of_hbm_peak": round(cres["alg_bytes"] / csm["wall_s"] / 1e9 / HBM_PEAK_GBS, 4),
                   "kernel_us_per_step": round(csm["ev_mean_s"] * 1e6, 2)}
        log(f"chained step: {chained['us_per_step']:.1f} us ({chained['frac_of_hbm_peak']:.4f} of 8 TB/s)")
        del cres["ops"]
        torch.cuda.empty_cache()

    probe = read_probe_gbs(qd, torch, dev)
    log(f"read probe {probe:.0f} GB/s")
    # The timed kernel's average launch duration over the timed region: each
    # step's HIP-event pair on the launch stream brackets exactly one launch
    # of the persistent kernel (for the launch path: the step's launches and
    # the gaps between them).
    ksec = sm["ev_mean_s"]
    kernel_gbs = alg_bytes / ksec / 1e9
    persistent = res["persistent"]
    ngroups = res["ngroups"]
    if args.path == "plan" and not persistent:
        log("the plan replays per-group launches for this workload")
    family = ("small_m_int8_kernel" if m > 1 else f"gemv_int{8 if wl.fmt == 'int8_b32' else 4}_kernel")
    kname = ("stack_kernel (persistent, one launch per step)" if persistent else
             f"{family} family, {ngroups} fused launch{'es' if ngroups > 1 else ''} per step "
             f"(kernels plus launch gaps)")
    traffic = recorded_traffic("stack_kernel" if persistent else
                               ("small_m_launches" if m > 1 else "gemv_launches"), args.workload)
    out = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(wall_ms, 5),
        "us_per_step": round(wall_ms * 1e3, 2),
        "tok_per_s_equiv": round(m * 1e3 / wall_ms, 1),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": ("int8" if wl.fmt == "int8_b32" else "int4") + ("+fp16 head" if wl.head_fmt else ""),
        "data": "synthetic (W ~ N(0,0.02) fp32 quantized on the device; x ~ N(0,1) fp16)",
        "config": {"workload": args.workload, "m": m, "path": args.path,
                   "bytes_per_step": alg_bytes, "weight_bytes": res["weight_bytes"],
                   "projections": res["n_ops"],
                   "frac_of_hbm_peak": round(value / HBM_PEAK_GBS, 4),
                   "trials": TRIALS, "trials_us_per_step": sm["trials_us"], "trial_spread_us": sm["spread_us"],
                   "read_probe_gbs": round(probe, 1), "frac_of_read_probe": round(value / probe, 4),
                   "us_p10": round(sm["ev_p10_us"], 2), "us_p90": round(sm["ev_p90_us"], 2),
                   "glue": wl.glue, "chained": wl.chain or wl.glue,
                   "tok_per_s_note": ("linear stack with fused RMSNorm and SwiGLU glue; excludes attention, "
                                      "residual adds and embedding" if wl.glue else
                                      "linear stack only; excludes attention, norms and embedding")},
        "roofline": {"bound": "hbm", "achieved": round(kernel_gbs, 2), "peak": HBM_PEAK_GBS,
                     "unit": "GB/s", "frac": round(kernel_gbs / HBM_PEAK_GBS, 4),
                     "traffic": traffic, "kernel": kname,
                     "kernel_us_per_step": round(ksec * 1e6, 2)},
        "context": {"m4_max_decode_tok_s": M4_MAX_DECODE_TOK_S,
                    "note": "the pages' whole-model decode rates on Apple M4 Max (int8hu bundles); "
                            "another machine and a whole decoder, so context rather than a baseline"},
    }
    if wl.notes:
        out["config"]["note"] = wl.notes
    if chained is not None:
        out["config"]["chained_step"] = chained
    if res["per_step"] > 1:
        out["config"]["gemvs_per_step"] = res["per_step"]
        out["config"]["us_per_gemv"] = round(wall_ms * 1e3 / res["per_step"], 3)
    if not args.no_cpu_baseline:
        log("timing the CPU oracle over one full step")
        out["cpu_baseline"] = cpu_baseline(si, args.workload, alg_bytes // res["per_step"])
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
