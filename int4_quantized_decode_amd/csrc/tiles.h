// Device-side tile helpers shared by the GEMV, small-M and stack kernels:
// buffer-descriptor loads of the tiled blob and in-register dequantization.
#pragma once

#include "qd_internal.h"

namespace qd {

constexpr int kDescWord3 = 0x00020000;   // raw buffer, gfx9-family data format

__device__ __forceinline__ __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kDescWord3);
}

// Cache-policy bits of a buffer access on gfx950.
constexpr int kPolicyDefault = 0;
constexpr int kPolicyStream = 2;     // nt: weights are read once per step
constexpr int kPolicyCoherent = 16;  // sc1: coherent across the device's L2s

__device__ __forceinline__ u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicyDefault);
}

__device__ __forceinline__ u32x4 bload16_stream(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicyStream);
}

__device__ __forceinline__ u32x4 bload16_coherent(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, kPolicyCoherent);
}

__device__ __forceinline__ half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// sum_{i<8} q_i x_i for 8 int8 codes in (d0, d1) (k order) and 8 fp16 x.
// Each code byte b is biased to b ^ 0x80 = q + 128 and permuted under the
// fp16 exponent byte 0x64, giving the exact fp16 value 1024 + 128 + q; one
// packed subtraction of 1152 leaves q exactly.
__device__ __forceinline__ float dot8_int8(uint32_t d0, uint32_t d1, half8_t x, float acc) {
  const uint32_t u0 = d0 ^ 0x80808080u, u1 = d1 ^ 0x80808080u;
  const half2_t bias = {(half_t)-1152.0f, (half_t)-1152.0f};
  const half2_t q01 = as_h2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) + bias;
  const half2_t q23 = as_h2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) + bias;
  const half2_t q45 = as_h2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) + bias;
  const half2_t q67 = as_h2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) + bias;
  acc = __builtin_amdgcn_fdot2(q01, (half2_t){x[0], x[1]}, acc, false);
  acc = __builtin_amdgcn_fdot2(q23, (half2_t){x[2], x[3]}, acc, false);
  acc = __builtin_amdgcn_fdot2(q45, (half2_t){x[4], x[5]}, acc, false);
  acc = __builtin_amdgcn_fdot2(q67, (half2_t){x[6], x[7]}, acc, false);
  return acc;
}

// INT4 codes straight into fp16 operands with one AND per pair and no bias:
// a half whose exponent field is zero holds mantissa * 2^-24 exactly (an fp16
// subnormal), so for a word whose nibble p holds code (0,2,4,6,1,3,5,7)[p]
//   w        & 0x000F000F = half2(c0, c1) * 2^-24
//   w        & 0x00F000F0 = half2(c2, c3) * 2^-20   (16 times larger)
//   (w >> 8) & 0x000F000F = half2(c4, c5) * 2^-24
//   (w >> 8) & 0x00F000F0 = half2(c6, c7) * 2^-20
// The two kinds of pair accumulate apart (lo, hi); the caller forms
// lo + hi / 16 = 2^-24 sum c x, exact products summed in fp32.
__device__ __forceinline__ void dot8_int4_sub(uint32_t w, half8_t x, float& lo, float& hi) {
  const uint32_t m = 0x000F000Fu, m4 = 0x00F000F0u;
  const uint32_t w8 = w >> 8;
  lo = __builtin_amdgcn_fdot2(as_h2(w & m), (half2_t){x[0], x[1]}, lo, false);
  hi = __builtin_amdgcn_fdot2(as_h2(w & m4), (half2_t){x[2], x[3]}, hi, false);
  lo = __builtin_amdgcn_fdot2(as_h2(w8 & m), (half2_t){x[4], x[5]}, lo, false);
  hi = __builtin_amdgcn_fdot2(as_h2(w8 & m4), (half2_t){x[6], x[7]}, hi, false);
}

// Sum over the four lanes rho, rho+16, rho+32, rho+48 (a row's K quarters);
// lanes 0..15 end up holding their row's total.  Pure VALU lane swaps.
__device__ __forceinline__ float quad_reduce(float a) {
  const uint32_t u = __builtin_bit_cast(uint32_t, a);
  const auto r = __builtin_amdgcn_permlane32_swap(u, u, false, false);
  const float b = __builtin_bit_cast(float, (uint32_t)r[0]) + __builtin_bit_cast(float, (uint32_t)r[1]);
  const uint32_t ub = __builtin_bit_cast(uint32_t, b);
  const auto q = __builtin_amdgcn_permlane16_swap(ub, ub, false, false);
  return __builtin_bit_cast(float, (uint32_t)q[0]) + __builtin_bit_cast(float, (uint32_t)q[1]);
}

struct Tile8 {
  u32x4 c[4];
  u32x4 sc;
};

struct Tile4 {
  u32x4 c[2];
  u32x4 meta;
};

__device__ __forceinline__ Tile8 load_tile8(__amdgpu_buffer_rsrc_t r, int j, int lane) {
  const uint32_t t = (uint32_t)j * kTileBytes8;
  Tile8 T;
#pragma unroll
  for (int s = 0; s < 4; ++s) T.c[s] = bload16_stream(r, t + 1024 * s + 16 * lane);
  T.sc = bload16_stream(r, t + kMetaOffset8 + 16 * (lane & 15));
  return T;
}

__device__ __forceinline__ Tile4 load_tile4(__amdgpu_buffer_rsrc_t r, int j, int lane) {
  const uint32_t t = (uint32_t)j * kTileBytes4;
  Tile4 T;
#pragma unroll
  for (int s = 0; s < 2; ++s) T.c[s] = bload16_stream(r, t + 1024 * s + 16 * lane);
  T.meta = bload16_stream(r, t + kMetaOffset4 + 16 * (lane & 15));
  return T;
}

// Lane (g, rho)'s share of one int8 tile: row rho, K quarter g, 8 blocks.
__device__ __forceinline__ float tile_dot8(const Tile8& T, const half_t* xs_j, int g, float acc) {
  const half8_t scales = __builtin_bit_cast(half8_t, T.sc);
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const half8_t xv = *reinterpret_cast<const half8_t*>(xs_j + 64 * s + 32 * h + 8 * g);
      const float p = dot8_int8(T.c[s][2 * h], T.c[s][2 * h + 1], xv, 0.0f);
      acc = __builtin_fmaf((float)scales[2 * s + h], p, acc);
    }
  }
  return acc;
}

// Lane (g, rho)'s share of one int4 tile: 4 groups x 16 codes.
// y += sum_groups (s sum c x + m sum x); the code sums come out of
// dot8_int4_sub scaled by 2^-24, so the scale terms collect apart and take
// the factor 2^24 (exact) once per tile.
__device__ __forceinline__ float tile_dot4(const Tile4& T, const half_t* xs_j, const float* xsum_j, int g,
                                  float acc) {
  const half8_t meta = __builtin_bit_cast(half8_t, T.meta);
  const float4_t xsum = *reinterpret_cast<const float4_t*>(xsum_j + 4 * g);
  float acc_s = 0.0f;
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int gam = 2 * s + h;
      const half_t* xp = xs_j + 64 * gam + 16 * g;
      const half8_t xa = *reinterpret_cast<const half8_t*>(xp);
      const half8_t xb = *reinterpret_cast<const half8_t*>(xp + 8);
      float lo = 0.0f, hi = 0.0f;
      dot8_int4_sub(T.c[s][2 * h], xa, lo, hi);
      dot8_int4_sub(T.c[s][2 * h + 1], xb, lo, hi);
      acc_s = __builtin_fmaf((float)meta[gam], __builtin_fmaf(hi, 0.0625f, lo), acc_s);
      acc = __builtin_fmaf((float)meta[4 + gam], xsum[gam], acc);
    }
  }
  return __builtin_fmaf(acc_s, 16777216.0f, acc);
}

// fp16 weights (the unquantized head): chunk s holds the 32-wide block s of
// the super-block; lane (g, rho) has row rho's 8 values at 8g..8g+7.
struct Tile16 {
  u32x4 c[8];
};

__device__ __forceinline__ Tile16 load_tile16(__amdgpu_buffer_rsrc_t r, int j, int lane) {
  const uint32_t t = (uint32_t)j * kTileBytes16;
  Tile16 T;
#pragma unroll
  for (int s = 0; s < 8; ++s) T.c[s] = bload16_stream(r, t + 1024 * s + 16 * lane);
  return T;
}

// Lane (g, rho)'s share of one fp16 tile: row rho, 8 blocks x 8 values.
__device__ __forceinline__ float tile_dot16(const Tile16& T, const half_t* xs_j, int g, float acc) {
#pragma unroll
  for (int s = 0; s < 8; ++s) {
    const half8_t w = __builtin_bit_cast(half8_t, T.c[s]);
    const half8_t x = *reinterpret_cast<const half8_t*>(xs_j + 32 * s + 8 * g);
#pragma unroll
    for (int e = 0; e < 8; e += 2)
      acc = __builtin_amdgcn_fdot2((half2_t){w[e], w[e + 1]}, (half2_t){x[e], x[e + 1]}, acc, false);
  }
  return acc;
}

// 8 int8 codes (k order) -> 8 exact fp16 values.
__device__ __forceinline__ half8_t codes_to_half8(uint32_t d0, uint32_t d1) {
  const uint32_t u0 = d0 ^ 0x80808080u, u1 = d1 ^ 0x80808080u;
  const half2_t bias = {(half_t)-1152.0f, (half_t)-1152.0f};
  const half2_t q01 = as_h2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04010400u)) + bias;
  const half2_t q23 = as_h2(__builtin_amdgcn_perm(0x64646464u, u0, 0x04030402u)) + bias;
  const half2_t q45 = as_h2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04010400u)) + bias;
  const half2_t q67 = as_h2(__builtin_amdgcn_perm(0x64646464u, u1, 0x04030402u)) + bias;
  return (half8_t){q01[0], q01[1], q23[0], q23[1], q45[0], q45[1], q67[0], q67[1]};
}

}  // namespace qd
