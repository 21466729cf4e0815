// Decode-step stack driver: the layer's projections in dependency order
// ([q|k|v] -> o -> [gate|up] -> down per layer, then the LM head), each group
// of projections that share an activation fused into one launch, all on one
// stream.  The pages run decode as one static S=1 step per token that reads
// every weight once (zoo Qwen3-VL page, Measured paragraph; Core AI 4B/8B
// cards, Measured paragraph); this is that step's linear part.
#include <cstring>
#include <new>

#include "stack.h"

namespace qd {

namespace {

bool same_range_overlap(const void* a, uint64_t an, const void* b, uint64_t bn) {
  if (!a || !b || !an || !bn) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

}  // namespace

qd_status build_groups(const qd_linear_op* ops, int64_t n_ops, int64_t m,
                       std::vector<StackGroup>* out) {
  out->clear();
  if (m < 1 || m > QD_MAX_M) return QD_ESHAPE;
  if (n_ops < 0) return QD_EINVAL;
  if (n_ops > 0 && !ops) return QD_EINVAL;
  for (int64_t i = 0; i < n_ops; ++i) {
    qd_status st = validate_op(ops[i], m);
    if (st != QD_OK) return st;
  }
  int64_t i = 0;
  while (i < n_ops) {
    int64_t e = i + 1;
    while (e < n_ops && ops[e].group == ops[i].group) ++e;
    // Members of one group share x, K, format and prologue; their outputs are
    // disjoint and none of them overlaps the group's input.
    const uint64_t xbytes = (uint64_t)(ops[i].prologue == QD_PRO_GLU ? 2 : 1) * m * ops[i].w.k * 2;
    for (int64_t p = i; p < e; ++p) {
      if (ops[p].w.fmt != ops[i].w.fmt || ops[p].w.k != ops[i].w.k || ops[p].x != ops[i].x ||
          ops[p].prologue != ops[i].prologue || ops[p].gamma != ops[i].gamma ||
          memcmp(&ops[p].eps, &ops[i].eps, sizeof(float)) != 0)
        return QD_EINVAL;
      const uint64_t ybytes = (uint64_t)m * ops[p].w.n * 2;
      if (ops[p].w.k > 0 && same_range_overlap(ops[p].y, ybytes, ops[i].x, xbytes)) return QD_EINVAL;
      for (int64_t q = i; q < p; ++q)
        if (same_range_overlap(ops[p].y, ybytes, ops[q].y, (uint64_t)m * ops[q].w.n * 2))
          return QD_EINVAL;
    }
    StackGroup cur{};
    auto flush = [&]() {
      if (cur.args.n_mem > 0) out->push_back(cur);
      cur = StackGroup{};
    };
    for (int64_t p = i; p < e; ++p) {
      const qd_linear_op& op = ops[p];
      if (op.w.n == 0) continue;
      if (cur.args.n_mem == kMaxMembers) flush();
      LinearArgs& a = cur.args;
      cur.fmt = op.w.fmt;
      cur.zero_fill = op.w.k == 0;
      a.mem[a.n_mem] = Member{static_cast<const uint8_t*>(op.w.data), op.y, op.w.n, a.total_rg,
                              op.epilogue};
      a.total_rg += ceil_div(op.w.n, kTileRows);
      a.n_mem += 1;
      a.J = (int)ceil_div(op.w.k, kSuperK);
      a.k = op.w.k;
      a.x = op.x;
      a.m = (int)m;
      a.pro = op.prologue;
      a.gamma = op.gamma;
      a.eps = op.eps;
    }
    flush();
    i = e;
  }
  return QD_OK;
}

hipError_t launch_groups(const std::vector<StackGroup>& groups, hipStream_t s) {
  for (const StackGroup& g : groups) {
    hipError_t e;
    if (g.zero_fill) {
      e = hipSuccess;
      for (int i = 0; i < g.args.n_mem && e == hipSuccess; ++i)
        e = launch_fill_zero(g.args.mem[i].y, (int64_t)g.args.m * g.args.mem[i].n, s);
    } else if (g.args.m == 1) {
      e = launch_gemv(g.fmt, g.args, s);
    } else {
      e = launch_small_m(g.fmt, g.args, s);
    }
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace qd

