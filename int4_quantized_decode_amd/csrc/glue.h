// Element-wise glue fused into the projections: the RMSNorm prologue, the
// gated product prologue and the silu epilogue (the zoo Qwen3-VL page,
// Architecture paragraph, names a Qwen3 decoder with a SwiGLU MLP).  The
// formulas and fp16 storage points are the ones qdecode.h states for
// qd_prologue and qd_epilogue; every kernel family calls these helpers so
// the element-wise arithmetic is the same on every path.
#pragma once

#include "tiles.h"

namespace qd {

// silu of an fp16 gate value, in fp32, stored as fp16.  expf is accurate to
// about one ulp; a large negative argument makes exp overflow and the
// quotient a signed zero, a large positive one makes it the argument.
__device__ __forceinline__ half_t silu_h(half_t a) {
  const float v = (float)a;
  return (half_t)(v / (1.0f + expf(-v)));
}

// The stored output of an op: fp16 of the fp32 sum, then the epilogue.
__device__ __forceinline__ uint16_t epilogue_bits(float acc, int epi) {
  half_t v = (half_t)acc;
  if (epi == QD_EPI_SILU) v = silu_h(v);
  return __builtin_bit_cast(uint16_t, v);
}

// Gated product of 8 values: fp16 * fp16 rounded once (a packed fp16
// multiply is correctly rounded).  Whole vectors are reinterpreted: with this
// compiler a bit cast of one element v[i] of a vector read element 0.
__device__ __forceinline__ u32x4 glu8(u32x4 a, u32x4 b) {
  return __builtin_bit_cast(u32x4, __builtin_bit_cast(half8_t, a) * __builtin_bit_cast(half8_t, b));
}

// Sum of squares of 8 fp16 values added to acc, in a fixed order.
__device__ __forceinline__ float sumsq8(u32x4 v, float acc) {
  const half8_t h = __builtin_bit_cast(half8_t, v);
#pragma unroll
  for (int i = 0; i < 8; ++i) acc = __builtin_fmaf((float)h[i], (float)h[i], acc);
  return acc;
}

// r = 1 / sqrt(mean + eps), with correctly rounded fp32 division and root.
__device__ __forceinline__ float rms_inverse(float sumsq, int64_t k, float eps) {
  return 1.0f / sqrtf(sumsq / (float)k + eps);
}

// RMSNorm of 8 values: fp16(gamma * fp16(x * r)); the second product is of
// two fp16 values, rounded once.
__device__ __forceinline__ u32x4 rms8(u32x4 x, float r, u32x4 gamma) {
  const half8_t h = __builtin_bit_cast(half8_t, x);
  half8_t n;
#pragma unroll
  for (int i = 0; i < 8; ++i) n[i] = (half_t)((float)h[i] * r);
  return glu8(__builtin_bit_cast(u32x4, n), gamma);
}

// Wave-wide sum (every lane gets the total), in a fixed butterfly order.
__device__ __forceinline__ float wave_sum(float v) {
#pragma unroll
  for (int s = 32; s >= 1; s >>= 1) v += __shfl_xor(v, s);
  return v;
}

}  // namespace qd
