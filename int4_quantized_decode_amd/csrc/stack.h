// Decode-step stack driver (internal).
#pragma once

#include <vector>

#include "qd_internal.h"

namespace qd {

// One launch of the stack: up to kMaxMembers matrices sharing x.
struct StackGroup {
  int fmt;
  bool zero_fill;        // K == 0: outputs are zeros
  LinearArgs args;
};

qd_status validate_op(const qd_linear_op& op, int64_t m);
qd_status build_groups(const qd_linear_op* ops, int64_t n_ops, int64_t m,
                       std::vector<StackGroup>* out);
hipError_t launch_groups(const std::vector<StackGroup>& groups, hipStream_t s);

qd_status plan_create(const qd_linear_op* ops, int64_t n_ops, int64_t m, qd_stack_plan** out);
qd_status plan_run(qd_stack_plan* plan, hipStream_t s);
qd_status plan_error(qd_stack_plan* plan, int32_t* out_error);
bool plan_is_persistent(const qd_stack_plan* plan);
void plan_set_spin_limit(qd_stack_plan* plan, uint32_t polls);
void plan_destroy(qd_stack_plan* plan);
qd_status stack_run_noalloc(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t* err_flag,
                           hipStream_t s);
qd_status plan_describe(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t workgroups,
                        int64_t* out, int64_t cap, int64_t* out_len);

}  // namespace qd
