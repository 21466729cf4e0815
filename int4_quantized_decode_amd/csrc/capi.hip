// C ABI of libqdecode: host-side validation, then enqueue on the caller's
// stream.  Nothing here allocates except qd_stack_plan_create.
#include <cmath>
#include <cstddef>
#include <new>
#include <vector>

#include "qd_internal.h"
#include "stack.h"

#define QD_EXPORT extern "C" __attribute__((visibility("default")))

using namespace qd;

static_assert(sizeof(qd_linear_op) == 80 && offsetof(qd_linear_op, gamma) == 64 &&
                  offsetof(qd_linear_op, eps) == 72 && offsetof(qd_linear_op, epilogue) == 76,
              "qd_linear_op layout is part of the ABI");

namespace {

bool fmt_ok(int32_t f) { return f == QD_FMT_INT8_B32 || f == QD_FMT_INT4_G64 || f == QD_FMT_FP16; }
int64_t k_multiple(int32_t f) { return f == QD_FMT_INT4_G64 ? 64 : 32; }

bool overlaps(const void* a, uint64_t abytes, const void* b, uint64_t bbytes) {
  if (!a || !b || abytes == 0 || bbytes == 0) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bbytes && b0 < a0 + abytes;
}

qd_status check_shape(int32_t fmt, int64_t n, int64_t k) {
  if (!fmt_ok(fmt)) return QD_EINVAL;
  if (n < 0 || k < 0 || k % k_multiple(fmt) != 0 || k > QD_MAX_K) return QD_ESHAPE;
  if (ceil_div(n, kTileRows) > (int64_t)INT32_MAX) return QD_ESHAPE;
  return QD_OK;
}

qd_status check_weight(const qd_weight* w, int32_t want_fmt) {
  if (!w) return QD_EINVAL;
  if (!fmt_ok(w->fmt)) return QD_EINVAL;
  if (want_fmt && w->fmt != want_fmt) return QD_EFORMAT;
  qd_status st = check_shape(w->fmt, w->n, w->k);
  if (st != QD_OK) return st;
  if (w->n > 0 && w->k > 0) {
    if (!w->data) return QD_EINVAL;
    if ((uintptr_t)w->data % 16) return QD_EALIGN;
    if (w->bytes < qd_packed_bytes(w->fmt, w->n, w->k)) return QD_ESHAPE;
  }
  return QD_OK;
}

// x, y of one product with m token rows; x holds x_blocks blocks of m x K
// values (2 for a gated-product prologue).
qd_status check_io(const qd_weight* w, const uint16_t* x, const uint16_t* y, int64_t m,
                   int x_blocks = 1) {
  if (w->n == 0) return QD_OK;
  if (!y) return QD_EINVAL;
  if ((uintptr_t)y % 2) return QD_EALIGN;
  if (w->k == 0) return QD_OK;
  if (!x) return QD_EINVAL;
  if ((uintptr_t)x % 16) return QD_EALIGN;
  const uint64_t ybytes = (uint64_t)m * w->n * 2, xbytes = (uint64_t)x_blocks * m * w->k * 2;
  if (overlaps(y, ybytes, x, xbytes) || overlaps(y, ybytes, w->data, w->bytes)) return QD_EINVAL;
  return QD_OK;
}

LinearArgs single_args(const qd_weight* w, const uint16_t* x, uint16_t* y, int64_t m) {
  LinearArgs a{};
  a.mem[0] = Member{static_cast<const uint8_t*>(w->data), y, w->n, 0, QD_EPI_NONE};
  a.n_mem = 1;
  a.J = (int)ceil_div(w->k, kSuperK);
  a.k = w->k;
  a.total_rg = ceil_div(w->n, kTileRows);
  a.x = x;
  a.m = (int)m;
  return a;
}

qd_status to_status(hipError_t e) { return e == hipSuccess ? QD_OK : QD_ELAUNCH; }

qd_status run_linear(const qd_weight* w, const uint16_t* x, uint16_t* y, int64_t m,
                     hipStream_t s, bool small_m) {
  if (w->n == 0) return QD_OK;
  if (w->k == 0) return to_status(launch_fill_zero(y, m * w->n, s));
  const LinearArgs a = single_args(w, x, y, m);
  return to_status(small_m ? launch_small_m(w->fmt, a, s) : launch_gemv(w->fmt, a, s));
}

qd_status pack_common(int32_t fmt, const float* w, int64_t n, int64_t k, void* out,
                      uint64_t out_bytes, int32_t* err, void* stream) {
  qd_status st = check_shape(fmt, n, k);
  if (st != QD_OK) return st;
  const uint64_t need = qd_packed_bytes(fmt, n, k);
  if (need == 0) return QD_OK;
  if (!out) return QD_EINVAL;
  if (out_bytes < need) return QD_ESHAPE;
  if ((uintptr_t)out % 16) return QD_EALIGN;
  if (n > 0 && k > 0) {
    if (!w) return QD_EINVAL;
    if ((uintptr_t)w % 16) return QD_EALIGN;
    if (overlaps(out, need, w, (uint64_t)n * k * 4)) return QD_EINVAL;
  }
  hipStream_t s = static_cast<hipStream_t>(stream);
  uint8_t* o = static_cast<uint8_t*>(out);
  hipError_t e = fmt == QD_FMT_INT8_B32   ? launch_pack_int8(w, n, k, o, err, s)
                 : fmt == QD_FMT_INT4_G64 ? launch_pack_int4(w, n, k, o, err, s)
                                          : launch_pack_fp16(w, n, k, o, err, s);
  return to_status(e);
}

}  // namespace

QD_EXPORT uint64_t qd_packed_bytes(int32_t fmt, int64_t n, int64_t k) {
  if (check_shape(fmt, n, k) != QD_OK) return 0;
  return (uint64_t)ceil_div(n, kTileRows) * (uint64_t)ceil_div(k, kSuperK) * (uint64_t)tile_bytes(fmt);
}

QD_EXPORT const char* qd_status_string(int32_t status) {
  switch (status) {
    case QD_OK: return "ok";
    case QD_EINVAL: return "invalid argument (null pointer, unknown format, overlapping buffers or bad plan)";
    case QD_ESHAPE: return "invalid shape (K multiple, K limit, M range, or buffer too small)";
    case QD_EALIGN: return "misaligned pointer (blob, x and W need 16-byte alignment)";
    case QD_ERANGE: return "value out of range (non-finite weight or fp16 overflow of a scale)";
    case QD_ELAUNCH: return "HIP launch or runtime call failed";
    case QD_EFORMAT: return "weight format not supported by this entry point";
    case QD_EDEVICE: return "no usable device, or plan used on another device";
    default: return "unknown status";
  }
}

QD_EXPORT qd_status qpack_int8_b32(const float* w, int64_t n, int64_t k, void* out,
                                   uint64_t out_bytes, int32_t* err_flag, void* stream) {
  return pack_common(QD_FMT_INT8_B32, w, n, k, out, out_bytes, err_flag, stream);
}

QD_EXPORT qd_status qpack_int4_g64(const float* w, int64_t n, int64_t k, void* out,
                                   uint64_t out_bytes, int32_t* err_flag, void* stream) {
  return pack_common(QD_FMT_INT4_G64, w, n, k, out, out_bytes, err_flag, stream);
}

QD_EXPORT qd_status qpack_fp16(const float* w, int64_t n, int64_t k, void* out, uint64_t out_bytes,
                               int32_t* err_flag, void* stream) {
  return pack_common(QD_FMT_FP16, w, n, k, out, out_bytes, err_flag, stream);
}

QD_EXPORT qd_status qgemv_int8_b32(const qd_weight* w, const uint16_t* x, uint16_t* y,
                                   void* stream) {
  qd_status st = check_weight(w, QD_FMT_INT8_B32);
  if (st == QD_OK) st = check_io(w, x, y, 1);
  if (st != QD_OK) return st;
  return run_linear(w, x, y, 1, static_cast<hipStream_t>(stream), false);
}

QD_EXPORT qd_status qgemv_int4_g64(const qd_weight* w, const uint16_t* x, uint16_t* y,
                                   void* stream) {
  qd_status st = check_weight(w, QD_FMT_INT4_G64);
  if (st == QD_OK) st = check_io(w, x, y, 1);
  if (st != QD_OK) return st;
  return run_linear(w, x, y, 1, static_cast<hipStream_t>(stream), false);
}

QD_EXPORT qd_status qgemv_fp16(const qd_weight* w, const uint16_t* x, uint16_t* y, void* stream) {
  qd_status st = check_weight(w, QD_FMT_FP16);
  if (st == QD_OK) st = check_io(w, x, y, 1);
  if (st != QD_OK) return st;
  return run_linear(w, x, y, 1, static_cast<hipStream_t>(stream), false);
}

QD_EXPORT qd_status qgemm_small_m(const qd_weight* w, const uint16_t* x, uint16_t* y, int64_t m,
                                  void* stream) {
  qd_status st = check_weight(w, 0);
  if (st != QD_OK) return st;
  if (m < 1 || m > QD_MAX_M) return QD_ESHAPE;
  st = check_io(w, x, y, m);
  if (st != QD_OK) return st;
  return run_linear(w, x, y, m, static_cast<hipStream_t>(stream), true);
}

QD_EXPORT qd_status decode_linear_stack(const qd_linear_op* ops, int64_t n_ops, int64_t m,
                                        void* stream) {
  std::vector<StackGroup> groups;
  qd_status st = build_groups(ops, n_ops, m, &groups);
  if (st != QD_OK) return st;
  return to_status(launch_groups(groups, static_cast<hipStream_t>(stream)));
}

QD_EXPORT qd_status qd_stack_plan_create(const qd_linear_op* ops, int64_t n_ops, int64_t m,
                                         qd_stack_plan** out) {
  if (!out) return QD_EINVAL;
  *out = nullptr;
  return plan_create(ops, n_ops, m, out);
}

QD_EXPORT qd_status qd_stack_plan_run(qd_stack_plan* plan, void* stream) {
  if (!plan) return QD_EINVAL;
  return plan_run(plan, static_cast<hipStream_t>(stream));
}

QD_EXPORT qd_status qd_stack_plan_error(qd_stack_plan* plan, int32_t* out_error) {
  if (!plan || !out_error) return QD_EINVAL;
  return plan_error(plan, out_error);
}

QD_EXPORT qd_status qd_read_probe(const void* buf, uint64_t bytes, void* sink, int32_t grid,
                                  void* stream) {
  if (!buf || !sink) return QD_EINVAL;
  if ((reinterpret_cast<uintptr_t>(buf) & 15) || (reinterpret_cast<uintptr_t>(sink) & 3)) return QD_EALIGN;
  if (bytes == 0 || grid < 1 || grid > 65535) return QD_ESHAPE;
  if (qd::launch_read_probe(buf, bytes, static_cast<uint32_t*>(sink), grid,
                            static_cast<hipStream_t>(stream)) != hipSuccess)
    return QD_ELAUNCH;
  return QD_OK;
}

QD_EXPORT qd_status qd_stack_plan_is_persistent(const qd_stack_plan* plan, int32_t* out) {
  if (!plan || !out) return QD_EINVAL;
  *out = plan_is_persistent(plan) ? 1 : 0;
  return QD_OK;
}

QD_EXPORT qd_status qd_stack_plan_set_spin_limit(qd_stack_plan* plan, uint32_t polls) {
  if (!plan) return QD_EINVAL;
  plan_set_spin_limit(plan, polls);
  return QD_OK;
}

QD_EXPORT void qd_stack_plan_destroy(qd_stack_plan* plan) { plan_destroy(plan); }

QD_EXPORT qd_status qd_stack_run_noalloc(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t* err_flag,
                                         void* stream) {
  return stack_run_noalloc(ops, n_ops, m, err_flag, static_cast<hipStream_t>(stream));
}

QD_EXPORT qd_status qd_stack_plan_describe(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t workgroups,
                                           int64_t* out, int64_t cap, int64_t* out_len) {
  if (!out_len || cap < 0) return QD_EINVAL;
  return plan_describe(ops, n_ops, m, workgroups, out, cap, out_len);
}

// ---- validation helpers shared with stack.hip --------------------------------

namespace qd {

qd_status validate_op(const qd_linear_op& op, int64_t m) {
  qd_status st = check_weight(&op.w, 0);
  if (st != QD_OK) return st;
  if (op.epilogue != QD_EPI_NONE && op.epilogue != QD_EPI_SILU) return QD_EINVAL;
  if (op.prologue == QD_PRO_RMSNORM) {
    if (!(std::isfinite(op.eps) && op.eps > 0.0f)) return QD_EINVAL;
    if (op.w.n > 0 && op.w.k > 0) {
      if (!op.gamma) return QD_EINVAL;
      if ((uintptr_t)op.gamma % 16) return QD_EALIGN;
      if (overlaps(op.y, (uint64_t)m * op.w.n * 2, op.gamma, (uint64_t)op.w.k * 2)) return QD_EINVAL;
    }
  } else if (op.prologue == QD_PRO_NONE || op.prologue == QD_PRO_GLU) {
    if (op.gamma || op.eps != 0.0f) return QD_EINVAL;
  } else {
    return QD_EINVAL;
  }
  return check_io(&op.w, op.x, op.y, m, op.prologue == QD_PRO_GLU ? 2 : 1);
}

}  // namespace qd
