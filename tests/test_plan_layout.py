"""Host-side checks of the persistent step's schedule (no GPU needed).

qd_stack_plan_describe returns the tables qd_stack_plan_create builds, from
the host alone.  These tests build decode-step op lists with synthetic
addresses (the pointers are only compared and offset) and check the tables
against properties stated here independently of the library:

* every output row of every op in the persistent prefix is computed exactly
  once, by one member slice, and the replayed tail starts where it should;
* each group's members tile its row-groups in order, and each group's
  row-groups are split over the workgroups as one contiguous range each,
  disjoint and covering, with tile offsets that are running sums;
* boundary ordering: a group may stage early exactly when no earlier group
  writes its activation (or RMSNorm weight); a group acknowledges its stores
  exactly when a later group reads them or overwrites them; later row ranges
  of a split group wait for nothing; reading through the caches only where
  one step group writes the lines and nothing brought them in before;
* at several token rows, the activation copies: slots disjoint and sized for
  the matrix-core order, one copy job per activation no group writes, and an
  op's outputs copied only when they are exactly a later group's activation,
  at offsets that stay valid under the row-range split;
* the LDS the kernel asks for fits one CU (160 KiB).
"""
import ctypes
from dataclasses import dataclass

import pytest

from synthetic_inputs import QWEN3_2B, QWEN3_8B, QWEN38_27B, Decoder

FMT = {"int8_b32": 1, "int4_g64": 2, "fp16": 3}
PRO_NONE, PRO_RMSNORM, PRO_GLU = 0, 1, 2
EPI_NONE, EPI_SILU = 0, 1
EARLY, ACK, NOWAIT, CLEAN, PAIRED, INDEPENDENT, DYNAMIC = 1, 2, 4, 8, 16, 32, 64
TILE_BYTES = {1: 4352, 2: 2304}
LDS_MAX = 160 * 1024


@pytest.fixture(scope="module")
def L():
    from int4_quantized_decode_amd import _lib
    return _lib


class Heap:
    """Bump allocator of synthetic device addresses."""

    def __init__(self):
        self.top = 1 << 36

    def take(self, nbytes, align=4096):
        self.top = (self.top + align - 1) // align * align
        p = self.top
        self.top += max(nbytes, 1)
        return p


@dataclass
class Op:
    fmt: int
    n: int
    k: int
    data: int
    nbytes: int
    x: int
    y: int
    group: int
    pro: int = PRO_NONE
    gamma: int = 0
    eps: float = 0.0
    epi: int = EPI_NONE


class StepBuilder:
    def __init__(self, L, m):
        self.L, self.m, self.heap, self.ops, self.gid = L, m, Heap(), [], 0

    def act(self, k):
        return self.heap.take(self.m * k * 2)

    def group(self, members, x, fmt, pro=PRO_NONE, gamma=0, epis=None, ys=None):
        """members: [(n, k)]; returns the output addresses."""
        out = []
        for i, (n, k) in enumerate(members):
            nb = self.L.lib.qd_packed_bytes(fmt, n, k)
            y = ys[i] if ys else self.heap.take(self.m * n * 2)
            self.ops.append(Op(fmt, n, k, self.heap.take(nb), nb, x, y, self.gid, pro, gamma,
                               1e-6 if pro == PRO_RMSNORM else 0.0,
                               epis[i] if epis else EPI_NONE))
            out.append(y)
        self.gid += 1
        return out

    def array(self):
        arr = (self.L.QDLinearOp * len(self.ops))()
        for i, o in enumerate(self.ops):
            w = self.L.QDWeight(o.fmt, 0, o.n, o.k, o.data, o.nbytes)
            arr[i] = self.L.QDLinearOp(w, o.x, o.y, o.group, o.pro, o.gamma or None, o.eps, o.epi)
        return arr


def step_ops(L, dec: Decoder, m, fmt, layers=None, chain=False, glue=False, head_fmt=None):
    """One decode step's op list: q|k|v -> o -> gate|up -> down per layer,
    then the head.  Plain: every group reads an activation of its own.
    Chained: each group reads an earlier group's output.  Glued:
    RMSNorm before q|k|v, gate|up and the head, silu on gate, the
    gated product before down."""
    b = StepBuilder(L, m)
    H, Q, KV, I = dec.hidden, dec.q_dim, dec.kv_dim, dec.mlp
    f = FMT[fmt]
    h = b.act(H)
    for _ in range(dec.layers if layers is None else layers):
        if glue:
            g1, g2, g3 = (b.heap.take(H * 2) for _ in range(3))
            q, _, _ = b.group([(Q, H), (KV, H), (KV, H)], h, f, PRO_RMSNORM, g1)
            o, = b.group([(H, Q)], q, f)
            gu = b.heap.take(m * 2 * I * 2)
            b.group([(I, H), (I, H)], o, f, PRO_RMSNORM, g2, epis=[EPI_SILU, EPI_NONE],
                    ys=[gu, gu + m * I * 2])
            h, = b.group([(H, I)], gu, f, PRO_GLU)
            hg = g3
        elif chain:
            q, _, _ = b.group([(Q, H), (KV, H), (KV, H)], h, f)
            o, = b.group([(H, Q)], q, f)
            g, _ = b.group([(I, H), (I, H)], o, f)
            h, = b.group([(H, I)], g, f)
        else:
            b.group([(Q, H), (KV, H), (KV, H)], b.act(H), f)
            b.group([(H, Q)], b.act(Q), f)
            b.group([(I, H), (I, H)], b.act(H), f)
            b.group([(H, I)], b.act(I), f)
            h = b.act(H)
    hf = FMT[head_fmt or fmt]
    if glue:
        b.group([(dec.vocab, H)], h, hf, PRO_RMSNORM, hg)
    else:
        b.group([(dec.vocab, H)], h, hf)
    return b


def describe(L, b, workgroups=256):
    arr = b.array()
    n = ctypes.c_int64(0)
    st = L.lib.qd_stack_plan_describe(arr, len(b.ops), b.m, workgroups, None, 0, ctypes.byref(n))
    assert st == 0, L.lib.qd_status_string(st)
    buf = (ctypes.c_int64 * n.value)()
    assert L.lib.qd_stack_plan_describe(arr, len(b.ops), b.m, workgroups, buf, n.value,
                                        ctypes.byref(n)) == 0
    v = list(buf)
    keys = ["version", "persistent", "fmt", "m", "glue", "prefix", "ngroups", "nmem", "G",
            "xt_total", "njobs", "lds", "x_bytes", "red_bytes", "cnt_bytes", "tab_bytes", "ss_total", "lag",
            "dyn_c", "dyn_q", "dyn_nch", "dyn_max"]
    d = dict(zip(keys, v[:len(keys)]))
    pos = len(keys)

    def take(count, width, names):
        nonlocal pos
        out = []
        for _ in range(count):
            out.append(dict(zip(names, v[pos:pos + width])))
            pos += width
        return out

    d["groups"] = take(d["ngroups"], 12, ["x", "gamma", "k", "J", "R", "mem0", "nmem", "pro", "order",
                                          "xt", "ss0", "ss_n"])
    d["members"] = take(d["nmem"], 8, ["blob", "y", "n", "rg_begin", "epi", "ld", "yt", "ss"])
    d["sched"] = take(d["ngroups"] * d["G"], 4, ["n", "off", "rg0", "nseg"])
    d["jobs"] = take(d["njobs"], 6, ["x", "t", "k", "first_block", "glu", "rec"])
    assert pos == len(v)
    return d


def overlap(a, an, b, bn):
    return an > 0 and bn > 0 and a < b + bn and b < a + an


def x_bytes(g, m):
    return m * g["k"] * 2 * (2 if g["pro"] == PRO_GLU else 1)


def attach_sources(b, d):
    """Map each member slice to its op: (op index, first row)."""
    by_blob = sorted((o.data, i) for i, o in enumerate(b.ops))
    src = []
    for mb in d["members"]:
        lo, hi = 0, len(by_blob) - 1
        while lo < hi:
            mid = (lo + hi + 1) // 2
            if by_blob[mid][0] <= mb["blob"]:
                lo = mid
            else:
                hi = mid - 1
        op_i = by_blob[lo][1]
        o = b.ops[op_i]
        J = -(-o.k // 256)
        skip, rem = divmod(mb["blob"] - o.data, J * TILE_BYTES[o.fmt])
        assert rem == 0 and 0 <= skip * 16 < o.n, "slice blob is not a row-group start of its op"
        assert mb["y"] == o.y + skip * 16 * 2, "slice y does not match its blob"
        assert mb["ld"] == o.n and mb["epi"] == o.epi
        src.append((op_i, skip * 16))
    return src


def check_dynamic(d, gi, g, m):
    """One token row, 3 GiB of weights or more, no group waiting for the one
    before it: the step's last group, with
    at least four row-groups per workgroup, is split at run time (DYNAMIC): no workgroup has a range
    in it, and workgroups claim chunks of C row-groups (about 32 per
    workgroup), dyn_q chunks ahead of their hand-outs (at least 64 tiles), at
    most dyn_max each.  Returns whether group gi is that group."""
    G = d["G"]
    dynamic = bool(g["order"] & DYNAMIC)
    waits = any(not h["order"] & NOWAIT for h in d["groups"][1:])
    expect = (m == 1 and gi == d["ngroups"] - 1 and g["R"] >= 4 * G and not g["order"] & PAIRED
              and d["weight_bytes"] >= 3 << 30 and not waits)
    assert dynamic == expect, f"group {gi}: dynamic flag"
    if not dynamic:
        return False
    sch = d["sched"][gi * G:(gi + 1) * G]
    assert all(s["n"] == 0 and s["nseg"] == 0 for s in sch)
    ju = -(-g["J"] // (2 if d["fmt"] == FMT["int4_g64"] else 1))
    c = max(1, g["R"] // (32 * G))
    nch = -(-g["R"] // c)
    q = -(-64 // (c * ju)) + 1
    assert (d["dyn_c"], d["dyn_nch"], d["dyn_q"]) == (c, nch, q)
    assert d["dyn_max"] == 4 * -(-nch // G) + q + 8 and d["dyn_max"] * G >= 4 * nch
    return True


def check_layout(b, d, lds_fits=True):
    m, ops = b.m, b.ops
    G, gs, ms = d["G"], d["groups"], d["members"]
    assert d["version"] == 4 and d["persistent"] == 1 and d["m"] == m
    src = attach_sources(b, d)

    # Rows: every op of the prefix is covered exactly once by its slices.
    rows = {i: [] for i in range(d["prefix"]) if ops[i].n > 0}
    for j, (op_i, r0) in enumerate(src):
        assert op_i < d["prefix"], "a replayed op appears in the persistent tables"
        rows[op_i].append((r0, r0 + ms[j]["n"]))
    for op_i, rs in rows.items():
        rs.sort()
        assert rs and rs[0][0] == 0 and rs[-1][1] == ops[op_i].n, f"op {op_i} not covered"
        assert all(rs[t][1] == rs[t + 1][0] for t in range(len(rs) - 1)), f"op {op_i} rows overlap/gap"

    for gi, g in enumerate(gs):
        mem = list(range(g["mem0"], g["mem0"] + g["nmem"]))
        assert mem and (gi == 0 or gs[gi - 1]["mem0"] + gs[gi - 1]["nmem"] == g["mem0"])
        rg = 0
        for j in mem:
            o = ops[src[j][0]]
            assert ms[j]["rg_begin"] == rg and o.x == g["x"] and o.k == g["k"] and o.pro == g["pro"]
            assert g["J"] == -(-o.k // 256) and g["gamma"] == o.gamma
            rg += -(-ms[j]["n"] // 16)
        assert rg == g["R"]
        d["weight_bytes"] = sum(-(-o.n // 16) * -(-o.k // 256) * TILE_BYTES[o.fmt] for o in ops[:d["prefix"]])
        if check_dynamic(d, gi, g, m):
            continue
        # Each workgroup one contiguous range; ranges cover [0, R) in
        # workgroup order, balanced within one row-group.  The order may
        # start at any workgroup (cyclically) where the row-groups do not
        # divide evenly, except in a paired group; otherwise at workgroup 0.
        sch = d["sched"][gi * G:(gi + 1) * G]

        def chain_from(rot):
            seq = [sch[(rot + i) % G] for i in range(G)]
            return (seq[0]["rg0"] == 0 and seq[-1]["rg0"] + seq[-1]["nseg"] == g["R"]
                    and all(seq[i]["rg0"] + seq[i]["nseg"] == seq[i + 1]["rg0"] for i in range(G - 1)))
        rots = [0] if (g["order"] & PAIRED or g["R"] % G == 0) else range(G)
        assert any(chain_from(r) for r in rots), f"group {gi}: ranges not in (cyclic) workgroup order"
        if g["order"] & PAIRED:
            # Paired (several token rows, its two members' gated product read
            # later): ranges of whole pairs of row-groups, balanced in pairs.
            assert m > 1 and g["nmem"] == 2 and g["R"] % 2 == 0
            assert all(s["rg0"] % 2 == 0 and s["nseg"] % 2 == 0 for s in sch)
            assert max(s["nseg"] for s in sch) - min(s["nseg"] for s in sch) <= 2
        else:
            assert max(s["nseg"] for s in sch) - min(s["nseg"] for s in sch) <= 1
        if m > 1:      # units of two row-groups at one super-block
            assert all(s["n"] == -(-s["nseg"] // 2) * g["J"] for s in sch)
        else:          # one token row: INT4 hands out two super-blocks at a time
            ku = 2 if d["fmt"] == FMT["int4_g64"] else 1
            assert all(s["n"] == s["nseg"] * -(-g["J"] // ku) for s in sch)
    # Tile offsets: running sums over the groups a workgroup has work in.
    for w in range(G):
        acc = 0
        for gi in range(len(gs)):
            s = d["sched"][gi * G + w]
            if s["nseg"]:
                assert s["off"] == acc
                acc += s["n"]

    # Boundary ordering.  The flags belong to the step's groups (one op
    # group, all its row ranges); the ranges of a split group each carry
    # them, and the ranges after the first also wait for nothing.
    def out_span(j):
        return ms[j]["y"], ((m - 1) * ms[j]["ld"] + ms[j]["n"]) * 2

    step_group = [ops[s[0]].group for s in src]
    sg = []                                   # [(group indices, member indices)]
    later = []                                # per plan group: a later row range of a split group
    for gi, g in enumerate(gs):
        later_range = gi > 0 and step_group[gs[gi - 1]["mem0"]] == step_group[g["mem0"]]
        later.append(later_range)
        if not later_range:
            sg.append(([], []))
        sg[-1][0].append(gi)
        sg[-1][1].extend(range(g["mem0"], g["mem0"] + g["nmem"]))

    def reads(g, j):
        return (overlap(g["x"], x_bytes(g, m), *out_span(j)) or
                (g["pro"] == PRO_RMSNORM and overlap(g["gamma"], g["k"] * 2, *out_span(j))))

    def lines(p, n):
        return (p & ~127, (p + n + 127) & ~127) if p and n else (0, 0)

    def hits(a, b):
        return a[0] < b[1] and b[0] < a[1]

    def acts(g):
        return [lines(g["x"], x_bytes(g, m)),
                lines(g["gamma"], g["k"] * 2) if g["pro"] == PRO_RMSNORM else (0, 0)]

    early = [not any(reads(gs[gl[0]], j) for _, mj in sg[:i] for j in mj) for i, (gl, _) in enumerate(sg)]

    # No device-wide wait before a later row range, nor before a step group
    # that reads nothing an earlier group writes and writes nothing an
    # earlier group reads or writes.
    def writes_into(mine, t):
        h = gs[sg[t][0][0]]
        return any(overlap(*out_span(a), h["x"], x_bytes(h, m)) or
                   (h["pro"] == PRO_RMSNORM and overlap(*out_span(a), h["gamma"], h["k"] * 2)) or
                   any(overlap(*out_span(a), *out_span(j)) for j in sg[t][1])
                   for a in mine)

    for i, (gi_list, mem) in enumerate(sg):
        independent = i > 0 and early[i] and not any(writes_into(mem, t) for t in range(i))
        for gi in gi_list:
            assert bool(gs[gi]["order"] & NOWAIT) == (later[gi] or independent), f"group {gi} no-wait flag"
            assert bool(gs[gi]["order"] & INDEPENDENT) == independent, f"group {gi} independent flag"
    for i, (gi_list, mem) in enumerate(sg):
        g = gs[gi_list[0]]
        e = early[i]
        ack = any(reads(gs[sg[t][0][0]], j) or
                  any(step_group[u] != step_group[j] and overlap(*out_span(u), *out_span(j)) for u in sg[t][1])
                  for t in range(i + 1, len(sg)) for j in mem)
        # Cache-read flag: one step group writes the activation's lines, and
        # no weight, no early read and no read up to that writer touches them.
        clean = False
        if not e:
            mine = acts(g)
            touch = lambda l: any(hits(l, a) for a in mine)
            writers, last = set(), -1
            for t in range(i):
                if any(touch(lines(*out_span(j))) for j in sg[t][1]):
                    writers.add(t)
                    last = t
            clean = len(writers) <= 1
            for t, (gl, mj) in enumerate(sg):
                h = gs[gl[0]]
                if any(touch(lines(ms[j]["blob"], -(-ms[j]["n"] // 16) * h["J"] * TILE_BYTES[d["fmt"]]))
                       for j in mj):
                    clean = False
                if t != i and (early[t] or t <= last) and any(touch(a) for a in acts(h)):
                    clean = False
        for gi in gi_list:
            o = gs[gi]["order"]
            assert bool(o & EARLY) == e, f"group {gi} early flag"
            assert bool(o & ACK) == ack, f"group {gi} acknowledge flag"
            assert bool(o & CLEAN) == clean, f"group {gi} cache-read flag"

    # Activation copies and sum-of-squares records (several token rows).
    if m == 1:
        assert d["xt_total"] == 0 and d["njobs"] == 0 and d["ss_total"] == 0
        assert all(g["xt"] == -1 and g["ss_n"] == 0 for g in gs)
        assert all(mb["yt"] == -1 and mb["ss"] == -1 for mb in ms)
        assert not any(g["order"] & PAIRED for g in gs)
    else:
        check_records(b, d, src, sg)
        slots = {}
        for g in gs:
            if g["xt"] >= 0:
                size = -(-g["J"] * 8192 // 256) * 256
                assert slots.setdefault(g["xt"], size) == size
        spans = sorted(slots.items())
        assert all(a + s <= b2 for (a, s), (b2, _) in zip(spans, spans[1:]))
        assert not spans or spans[-1][0] + spans[-1][1] <= d["xt_total"]
        # Jobs made before the step: copies (of x, or of the gated product of
        # its two blocks) and sum-of-squares records, one of each per key.
        for jb in d["jobs"]:
            assert (jb["t"] >= 0) != (jb["rec"] >= 0) and (jb["glu"] == 0 or jb["t"] >= 0)
        copy_jobs = {(jb["x"], jb["k"], jb["glu"]): jb["t"] for jb in d["jobs"] if jb["t"] >= 0}
        rec_jobs = {(jb["x"], jb["k"]): jb["rec"] for jb in d["jobs"] if jb["t"] < 0}
        assert len(copy_jobs) + len(rec_jobs) == d["njobs"]
        blocks = 0
        for jb in d["jobs"]:
            assert jb["first_block"] == blocks
            blocks += 2 * -(-jb["k"] // 256) if jb["t"] >= 0 else 1
        for gi, g in enumerate(gs):
            if g["order"] & EARLY:
                assert g["xt"] == copy_jobs[(g["x"], g["k"], int(g["pro"] == PRO_GLU))]
            if g["pro"] == PRO_GLU:
                assert g["xt"] >= 0, "a gated product at several token rows is read from its copy"
        # Output copies: member slices of one op share the op's copy, at
        # 512 bytes per row-group of skip, with skip whole 256-row blocks.
        base = {}
        for j, mb in enumerate(ms):
            if mb["yt"] < 0:
                continue
            op_i, r0 = src[j]
            assert r0 % 256 == 0, "copy offset cut inside a 256-row block"
            b0 = base.setdefault(op_i, mb["yt"] - r0 * 32)
            assert mb["yt"] == b0 + r0 * 32
        paired_op = {src[j][0]: bool(g["order"] & PAIRED) for g in gs
                     for j in range(g["mem0"], g["mem0"] + g["nmem"])}
        for g in gs:
            if g["order"] & PAIRED:   # the first member's copy slot holds the product, the second has none
                assert ms[g["mem0"] + 1]["yt"] == -1
        for op_i, b0 in base.items():
            o = ops[op_i]
            consumers = [g for g in gs if g["xt"] == b0]
            assert consumers and all(g["x"] == o.y and g["k"] == o.n for g in consumers)
            if paired_op[op_i]:
                assert all(g["pro"] == PRO_GLU for g in consumers)
            else:
                assert all(g["pro"] in (PRO_NONE, PRO_RMSNORM) for g in consumers)
            assert all(not (g["order"] & EARLY) for g in consumers)
        for g in gs:
            if g["xt"] >= 0 and not g["order"] & EARLY:
                assert g["xt"] in base.values()
    # (With few workgroups a group's partials outgrow one CU's LDS; the plan
    # then replays launches, which the device check in plan creation decides.)
    assert d["lds"] <= LDS_MAX or not lds_fits
    assert d["lds"] >= d["x_bytes"] + d["red_bytes"] + d["cnt_bytes"] + d["tab_bytes"]


def check_records(b, d, src, sg):
    """Several token rows: each RMSNorm group's ss_n records add up to its
    activation's per-token sums of squares.  Either no group of the step
    writes the activation and one record is made before the step (a record
    job on (x, K)), or the activation is exactly the whole output of one op
    that its last writer ran, and the records are that op's: G per member
    slice (one per workgroup), contiguous in slice order.  Records are
    disjoint and within ss_total; records nobody reads are never written."""
    m, ops, G, gs, ms = b.m, b.ops, d["G"], d["groups"], d["members"]
    rec_jobs = {(jb["x"], jb["k"]): jb["rec"] for jb in d["jobs"] if jb["t"] < 0}
    spans = sorted([(mb["ss"], G) for mb in ms if mb["ss"] >= 0] + [(r, 1) for r in rec_jobs.values()])
    assert all(a + n <= b2 for (a, n), (b2, _) in zip(spans, spans[1:]))
    assert sum(n for _, n in spans) == d["ss_total"]
    step_of = {}                                # plan group -> index into sg
    for i, (gl, _) in enumerate(sg):
        for gi in gl:
            step_of[gi] = i
    readers = set()
    for gi, g in enumerate(gs):
        if g["pro"] != PRO_RMSNORM:
            assert g["ss_n"] == 0
            continue
        writers = [t for t in range(step_of[gi]) for j in sg[t][1]
                   if overlap(g["x"], m * g["k"] * 2, ms[j]["y"], ((m - 1) * ms[j]["ld"] + ms[j]["n"]) * 2)]
        if not writers:
            assert (g["ss0"], g["ss_n"]) == (rec_jobs[(g["x"], g["k"])], 1)
            continue
        last = max(writers)
        mine = [j for j in sg[last][1] if ops[src[j][0]].y == g["x"]]
        assert mine, "RMSNorm records from an op that is not x's last writer"
        op_i = src[mine[0]][0]
        assert ops[op_i].n == g["k"] and all(src[j][0] == op_i for j in mine)
        assert [ms[j]["ss"] for j in mine] == [g["ss0"] + G * t for t in range(len(mine))]
        assert g["ss_n"] == G * len(mine)
        readers.update(mine)
    assert readers == {j for j, mb in enumerate(ms) if mb["ss"] >= 0}, "records nobody reads"
    for gl, mj in sg:
        assert len({src[j][0] for j in mj if ms[j]["ss"] >= 0}) <= 1, "two ops of one group with records"
        if gs[gl[0]]["order"] & PAIRED:
            assert all(ms[j]["ss"] < 0 for j in mj)


CASES = [
    ("qwen3-8b int8 m1", QWEN3_8B, 1, "int8_b32", {}),
    ("qwen3-8b int4 m1", QWEN3_8B, 1, "int4_g64", {}),
    ("qwen3-2b int8 m1", QWEN3_2B, 1, "int8_b32", {}),
    ("qwen3-8b int8 m16", QWEN3_8B, 16, "int8_b32", {}),
    ("qwen3-8b int4 m16", QWEN3_8B, 16, "int4_g64", {}),
    ("qwen3-8b int4 chain m3", QWEN3_8B, 3, "int4_g64", {"chain": True, "layers": 4}),
    ("qwen3-8b int8 chain m1", QWEN3_8B, 1, "int8_b32", {"chain": True}),
    ("qwen3-8b int8 chain m16", QWEN3_8B, 16, "int8_b32", {"chain": True}),
    ("qwen3-8b int8 glue m1", QWEN3_8B, 1, "int8_b32", {"glue": True}),
    ("qwen3-8b int8 glue m16", QWEN3_8B, 16, "int8_b32", {"glue": True}),
    ("qwen3-8b int4 glue m16", QWEN3_8B, 16, "int4_g64", {"glue": True}),
    ("qwen3-2b int8 glue m5", QWEN3_2B, 5, "int8_b32", {"glue": True}),
    ("qwen3.8-27b int8 glue m16 (3 layers)", QWEN38_27B, 16, "int8_b32", {"glue": True, "layers": 3}),
    ("qwen3.8-27b int8 m16 (4 layers)", QWEN38_27B, 16, "int8_b32", {"layers": 4}),
    ("qwen3.8-27b int8 chain m16 (3 layers)", QWEN38_27B, 16, "int8_b32", {"layers": 3, "chain": True}),
    ("qwen3-8b int8 chain m5", QWEN3_8B, 5, "int8_b32", {"chain": True, "layers": 4}),
    ("qwen3.8-27b int8 m1", QWEN38_27B, 1, "int8_b32", {}),
]


def expected_lag(b, d):
    """The drift bound the plan states: 16 groups from 12 GiB of weights in
    the persistent part, else none."""
    wbytes = sum(-(-o.n // 16) * -(-o.k // 256) * TILE_BYTES[o.fmt] for o in b.ops[:d["prefix"]])
    return 16 if wbytes >= 12 << 30 else 0


@pytest.mark.parametrize("name,dec,m,fmt,kw", CASES, ids=[c[0] for c in CASES])
def test_plan_layout_invariants(L, name, dec, m, fmt, kw):
    b = step_ops(L, dec, m, fmt, **kw)
    d = describe(L, b)
    assert d["prefix"] == len(b.ops) and d["glue"] == int(bool(kw.get("glue")))
    assert d["lag"] == expected_lag(b, d)
    check_layout(b, d)


def test_plan_layout_independent_groups(L):
    """The metric's workload (every group reads an activation of its own and
    writes fresh outputs): every group after the first is independent and
    waits for nothing; in the chained step none is."""
    d = describe(L, step_ops(L, QWEN3_8B, 1, "int8_b32"))
    assert all(g["order"] & INDEPENDENT and g["order"] & NOWAIT for g in d["groups"][1:])
    assert not d["groups"][0]["order"] & (INDEPENDENT | NOWAIT) and d["lag"] == 0
    d = describe(L, step_ops(L, QWEN3_8B, 1, "int8_b32", chain=True))
    assert not any(g["order"] & (INDEPENDENT | NOWAIT) for g in d["groups"])


@pytest.mark.parametrize("workgroups", [1, 7, 80, 255, 304, 512])
def test_plan_layout_other_workgroup_counts(L, workgroups):
    for m, kw in ((1, {"chain": True}), (16, {"chain": True}), (16, {})):
        b = step_ops(L, QWEN3_8B, m, "int8_b32", layers=2, **kw)
        d = describe(L, b, workgroups)
        assert d["G"] == workgroups
        check_layout(b, d, lds_fits=workgroups >= 80)


def test_plan_layout_fp16_head_is_replayed_tail(L):
    b = step_ops(L, QWEN3_2B, 1, "int8_b32", layers=3, head_fmt="fp16")
    d = describe(L, b)
    assert d["persistent"] == 1 and d["prefix"] == len(b.ops) - 1
    check_layout(b, d)


@pytest.mark.parametrize("m,fmt,kw", [(1, "fp16", {}), (16, "fp16", {})])
def test_plan_layout_replays_whole(L, m, fmt, kw):
    b = step_ops(L, QWEN3_8B, m, fmt, layers=1, **kw)
    d = describe(L, b)
    assert d["persistent"] == 0 and d["ngroups"] == 0 and len(d) == 22 + 4


def test_plan_layout_copy_not_cut_inside_a_block(L):
    """A producing member starting 4 row-groups into a group long enough to
    be split: with 8 workgroups the cuts come every 48 row-groups, 44 into
    the member first, so it writes no copy and its consumer reads its
    activation in place.  With the producer first the cuts fall at whole
    256-row blocks of it and the copy is kept."""
    b = StepBuilder(L, 16)
    x = b.act(4096)
    _, q = b.group([(64, 4096), (4096, 4096)], x, 1)
    b.group([(512, 4096)], q, 1)
    d = describe(L, b, 8)
    check_layout(b, d)
    assert d["groups"][0]["R"] < 260 and len(d["groups"]) > 2      # split into row ranges
    assert all(mb["yt"] == -1 for mb in d["members"])
    assert d["groups"][-1]["xt"] == -1
    b = StepBuilder(L, 16)
    x = b.act(4096)
    q, _ = b.group([(4096, 4096), (64, 4096)], x, 1)
    b.group([(512, 4096)], q, 1)
    d = describe(L, b, 8)
    check_layout(b, d)
    assert any(mb["yt"] >= 0 for mb in d["members"]) and d["groups"][-1]["xt"] >= 0


def test_plan_describe_errors(L):
    b = step_ops(L, QWEN3_2B, 1, "int8_b32", layers=1)
    arr, n = b.array(), ctypes.c_int64(0)
    lib = L.lib
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 1, 256, None, 0, None) == 1
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 1, 0, None, 0, ctypes.byref(n)) == 1
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 1, 513, None, 0, ctypes.byref(n)) == 1
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 1, 256, None, -1, ctypes.byref(n)) == 1
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 17, 256, None, 0, ctypes.byref(n)) == 2
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 1, 256, None, 0, ctypes.byref(n)) == 0
    need = n.value
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 1, 256, None, need + 100, ctypes.byref(n)) == 0
    assert n.value == need
    small = (ctypes.c_int64 * 4)()
    assert lib.qd_stack_plan_describe(arr, len(b.ops), 1, 256, small, 4, ctypes.byref(n)) == 2
    assert n.value == need and list(small) == [0, 0, 0, 0]


def test_plan_layout_copy_cuts_on_256_workgroups(L):
    """The layout the GPU test of the same name runs: at K = 5120 the split
    comes every 1024 row-groups; b (starting 4 row-groups in) is cut 1020
    row-groups in and writes no copy, d is cut at a whole block and both its
    slices write its copy, 1024 x 512 bytes apart."""
    b = StepBuilder(L, 16)
    x = b.act(5120)
    _, yb = b.group([(64, 5120), (24576, 5120)], x, 1)
    b.group([(512, 24576)], yb, 1)
    yd, _ = b.group([(24576, 5120), (64, 5120)], x, 1)
    b.group([(512, 24576)], yd, 1)
    d = describe(L, b, 256)
    check_layout(b, d)
    gs, ms = d["groups"], d["members"]
    assert [g["R"] for g in gs] == [1024, 516, 32, 1024, 516, 32]
    assert gs[2]["xt"] == -1 and gs[5]["xt"] >= 0
    d_slices = [mb["yt"] for mb in ms if yd <= mb["y"] < yd + 24576 * 2]
    assert len(d_slices) == 2 and d_slices[0] == gs[5]["xt"] and d_slices[1] - d_slices[0] == 1024 * 512
    assert all(mb["yt"] == -1 for mb in ms if yb <= mb["y"] < yb + 24576 * 2)


def _random_step(L, rng):
    """A random valid step: groups of 1-3 members with random N and K; each
    group's activation is fresh, an earlier op's whole output (when its N
    matches K) or a slice of one; outputs are fresh or overwrite an earlier
    op's output of the same size."""
    fmt = int(rng.choice([1, 2]))
    m = int(rng.choice([1, 2, 5, 16]))
    b = StepBuilder(L, m)
    outs = []                               # (address, n) of earlier outputs
    for _ in range(int(rng.integers(1, 9))):
        k = int(rng.choice([256, 512, 1024, 1088, 2048, 4096]))
        if fmt == 2 and k % 64:
            k = 1024
        cands = [(y, n) for y, n in outs if n >= k]
        r = rng.random()
        if cands and r < 0.4:
            y, n = cands[int(rng.integers(len(cands)))]
            x = y if n == k or m > 1 else y + 2 * int(rng.integers(0, (n - k) // 8 + 1)) * 8
        else:
            x = b.act(k)
        members = [(int(rng.choice([16, 48, 100, 256, 1000, 4096, 6000])), k)
                   for _ in range(int(rng.integers(1, 4)))]
        ys = []
        for n, _ in members:
            same = [y for y, nn in outs if nn == n and not overlap(y, m * n * 2, x, m * k * 2)]
            if same and rng.random() < 0.2 and all(y not in ys for y in same[:1]):
                ys.append(same[0])
            else:
                ys.append(b.heap.take(m * n * 2))
        if len(set(ys)) != len(ys):
            ys = [b.heap.take(m * n * 2) for n, _ in members]
        got = b.group(members, x, fmt, ys=ys)
        outs.extend(zip(got, [n for n, _ in members]))
    return b


def test_plan_layout_random_steps(L):
    """200 random steps through the same invariants, at random workgroup
    counts.  Steps the validation rejects (an output overlapping its own
    group's input, say) are skipped."""
    import numpy as np
    rng = np.random.default_rng(20261203)
    checked = 0
    for _ in range(200):
        b = _random_step(L, rng)
        G = int(rng.choice([3, 8, 64, 80, 256, 304]))
        arr, n = b.array(), ctypes.c_int64(0)
        if L.lib.qd_stack_plan_describe(arr, len(b.ops), b.m, G, None, 0, ctypes.byref(n)) != 0:
            continue
        d = describe(L, b, G)
        if not d["persistent"]:
            continue
        check_layout(b, d, lds_fits=G >= 80)
        checked += 1
    assert checked >= 100


def _glue_prefix(b):
    """The first op the persistent kernel cannot take in a glued step at
    several token rows, by the rules the plan states: an RMSNorm group needs
    its activation unwritten by the step, or exactly the whole output of one
    op of its last writer (an op that is then the only one of its group with
    sum-of-squares records, in a group that is not paired); a gated product
    needs its two blocks unwritten by the step, or exactly the whole outputs
    of the two ops of its last writer, A's first (a group that then runs
    paired and has no records)."""
    m, ops = b.m, b.ops
    groups = []                                   # [(first op, [op indices])]
    for i, o in enumerate(ops):
        if groups and ops[groups[-1][1][0]].group == o.group:
            groups[-1][1].append(i)
        else:
            groups.append((i, [i]))
    paired, recs = set(), {}                      # group index; group index -> op with records
    for g, (first, mem) in enumerate(groups):
        o = ops[first]
        if o.pro == PRO_NONE:
            continue
        span = m * o.k * 2 * (2 if o.pro == PRO_GLU else 1)
        last = max((h for h in range(g) for j in groups[h][1]
                    if overlap(o.x, span, ops[j].y, m * ops[j].n * 2)), default=None)
        if last is None:
            continue
        lm = groups[last][1]
        if o.pro == PRO_RMSNORM:
            hit = [j for j in lm if overlap(o.x, span, ops[j].y, m * ops[j].n * 2)]
            ok = (len(hit) == 1 and ops[hit[0]].y == o.x and ops[hit[0]].n == o.k and last not in paired
                  and recs.get(last, hit[0]) == hit[0])
            if ok:
                recs[last] = hit[0]
        else:
            ok = (len(lm) == 2 and last not in recs and ops[lm[0]].y == o.x and
                  ops[lm[1]].y == o.x + m * o.k * 2 and ops[lm[0]].n == o.k and ops[lm[1]].n == o.k)
            if ok:
                paired.add(last)
        if not ok:
            return first
    return len(ops)


def _random_glued_step(L, rng):
    """A random glued step at several token rows: groups take no prologue,
    RMSNorm or the gated product; activations are fresh, an earlier op's
    whole output, the start of a longer one, or (gated product) the two
    outputs of an earlier two-op group written A then B, B then A, or with
    a third op beside them; ops store with or without silu."""
    fmt = int(rng.choice([1, 2]))
    m = int(rng.choice([2, 5, 16]))
    b = StepBuilder(L, m)
    outs, pairs = [], []                          # (y, n); (A address, n) of two-op groups
    for _ in range(int(rng.integers(2, 8))):
        pro = int(rng.choice([PRO_NONE, PRO_RMSNORM, PRO_GLU]))
        k = int(rng.choice([256, 512, 1024, 2048]))
        r = rng.random()
        if pro == PRO_GLU and pairs and r < 0.6:
            x, k = pairs[int(rng.integers(len(pairs)))]
        elif pro != PRO_GLU and outs and r < 0.6:
            y, n = outs[int(rng.integers(len(outs)))]
            x, k = y, (n if rng.random() < 0.7 or n < 256 else 256)
        else:
            x = b.heap.take(m * k * 2 * (2 if pro == PRO_GLU else 1))
        gamma = b.heap.take(k * 2) if pro == PRO_RMSNORM else 0
        shape = rng.random()
        if shape < 0.35:                          # a gate|up-like pair writing one buffer
            n = int(rng.choice([256, 512, 1024]))
            gu = b.heap.take(2 * m * n * 2)
            ys = [gu, gu + m * n * 2] if rng.random() < 0.8 else [gu + m * n * 2, gu]
            members = [(n, k), (n, k)]
            if rng.random() < 0.15:
                members.append((64, k))
                ys.append(b.heap.take(m * 64 * 2))
            epis = [int(rng.choice([EPI_NONE, EPI_SILU])) for _ in members]
            got = b.group(members, x, fmt, pro, gamma, epis=epis, ys=ys)
            if len(members) == 2 and ys[0] < ys[1]:
                pairs.append((gu, n))
        else:
            members = [(int(rng.choice([64, 256, 512, 1024, 2048])), k) for _ in range(int(rng.integers(1, 4)))]
            epis = [int(rng.choice([EPI_NONE, EPI_SILU])) for _ in members]
            got = b.group(members, x, fmt, pro, gamma, epis=epis)
        outs.extend(zip(got, [n for n, _ in members]))
    return b


def test_plan_layout_random_glued_steps(L):
    """300 random glued steps at several token rows: the persistent part ends
    exactly where the rules say, and its tables pass every invariant above
    (records, paired groups, product copies included)."""
    import numpy as np
    rng = np.random.default_rng(20261204)
    checked = cut = 0
    for _ in range(300):
        b = _random_glued_step(L, rng)
        arr, n = b.array(), ctypes.c_int64(0)
        if L.lib.qd_stack_plan_describe(arr, len(b.ops), b.m, 256, None, 0, ctypes.byref(n)) != 0:
            continue
        d = describe(L, b, 256)
        want = _glue_prefix(b)
        if want == 0:
            assert d["persistent"] == 0
            continue
        assert d["persistent"] == 1 and d["prefix"] == want
        check_layout(b, d)
        checked += 1
        cut += want < len(b.ops)
    assert checked >= 150 and 20 <= cut <= checked - 20
