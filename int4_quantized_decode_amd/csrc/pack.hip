// Weight packers: fp32 [N, K] -> quantized codes + fp16 scales (+ mins) in the
// tiled layout, bit-exact with the quantizer definitions in qdecode.h.
//
// int8 b32: symmetric absmax per block of 32 (Qwen3-VL 4B/8B Core AI cards,
// Files table; zoo Qwen3.8-27B page, Numerics paragraph: absmax head rule, no
// clipping).  int4 g64: affine min/max per group of 64 (CoreML-LLM handoff
// page, Architecture paragraph, group_size 64).  fp16: the unquantized head of
// the int8lin variant (zoo Qwen3-VL page, Measured table, "2B int8lin (tied
// fp16 head)" row), round to nearest even.
//
// Bit-exactness rests on IEEE fp32 division rounded to nearest (the library is
// built with correctly rounded fp32 division, without fast-math), RNE
// float -> half conversion and round-half-even rintf.  Contraction is off
// here so no step is fused.
#include "qd_internal.h"

namespace qd {
namespace {

#pragma clang fp contract(off)

__device__ inline uint16_t half_bits(half_t h) { return __builtin_bit_cast(uint16_t, h); }

// One thread per (row-group r, super-block j, block beta in 0..7, row rho).
__global__ __launch_bounds__(256) void pack_int8_kernel(const float* __restrict__ w, int64_t n,
                                                        int64_t k, uint8_t* __restrict__ out,
                                                        int64_t J, int64_t total,
                                                        int32_t* __restrict__ err) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int rho = (int)(t & 15);
  const int beta = (int)((t >> 4) & 7);
  const int64_t rj = t >> 7;            // tile index r * J + j
  const int64_t j = rj % J;
  const int64_t r = rj / J;
  const int64_t row = r * kTileRows + rho;
  const int64_t k0 = j * kSuperK + beta * 32;
  uint8_t* tile = out + rj * kTileBytes8;

  uint32_t packed[8];                   // 32 codes, 4 per word, k order
#pragma unroll
  for (int i = 0; i < 8; ++i) packed[i] = 0u;
  uint16_t sbits = 0;

  if (row < n && k0 < k) {             // K % 32 == 0: a block is wholly in or out
    const float4_t* src = reinterpret_cast<const float4_t*>(w + row * k + k0);
    float v[32];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      float4_t f = src[i];
      v[4 * i + 0] = f[0];
      v[4 * i + 1] = f[1];
      v[4 * i + 2] = f[2];
      v[4 * i + 3] = f[3];
    }
    float a = 0.0f;
    bool finite = true;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
      finite = finite && __builtin_isfinite(v[i]);
      a = __builtin_fmaxf(a, __builtin_fabsf(v[i]));
    }
    const float s32 = a / 127.0f;
    const half_t s16 = (half_t)s32;
    const float sf = (float)s16;
    if (!finite || __builtin_isinf(sf)) {
      if (err) atomicOr(err, finite ? 2 : 1);
    } else {
      sbits = half_bits(s16);
      if (sf != 0.0f) {
#pragma unroll
        for (int i = 0; i < 32; ++i) {
          float q = __builtin_rintf(v[i] / sf);
          q = __builtin_fminf(__builtin_fmaxf(q, -127.0f), 127.0f);
          const uint32_t b = (uint32_t)(uint8_t)(int8_t)(int)q;
          packed[i >> 2] |= b << (8 * (i & 3));
        }
      }
    }
  }
  // Codes: block beta -> chunk s = beta / 2, half h = beta % 2; quarter g
  // holds k offsets 8g..8g+7 of the block at lane 16g + rho.
  const int s = beta >> 1, h = beta & 1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    u32x2 pair = {packed[2 * g], packed[2 * g + 1]};
    *reinterpret_cast<u32x2*>(tile + 1024 * s + 16 * (16 * g + rho) + 8 * h) = pair;
  }
  *reinterpret_cast<uint16_t*>(tile + kMetaOffset8 + 16 * rho + 2 * beta) = sbits;
}

// Nibble slot p of a word holds code k0 + kPerm4[p].
__constant__ int kPerm4[8] = {0, 2, 4, 6, 1, 3, 5, 7};

// One thread per (row-group r, super-block j, group gamma in 0..3, row rho).
__global__ __launch_bounds__(256) void pack_int4_kernel(const float* __restrict__ w, int64_t n,
                                                        int64_t k, uint8_t* __restrict__ out,
                                                        int64_t J, int64_t total,
                                                        int32_t* __restrict__ err) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int rho = (int)(t & 15);
  const int gamma = (int)((t >> 4) & 3);
  const int64_t rj = t >> 6;
  const int64_t j = rj % J;
  const int64_t r = rj / J;
  const int64_t row = r * kTileRows + rho;
  const int64_t k0 = j * kSuperK + gamma * 64;
  uint8_t* tile = out + rj * kTileBytes4;

  uint8_t q[64];
#pragma unroll
  for (int i = 0; i < 64; ++i) q[i] = 0;
  uint16_t sbits = 0, mbits = 0;

  if (row < n && k0 < k) {             // K % 64 == 0
    const float4_t* src = reinterpret_cast<const float4_t*>(w + row * k + k0);
    float v[64];
#pragma unroll
    for (int i = 0; i < 16; ++i) {
      float4_t f = src[i];
      v[4 * i + 0] = f[0];
      v[4 * i + 1] = f[1];
      v[4 * i + 2] = f[2];
      v[4 * i + 3] = f[3];
    }
    // IEEE 754-2019 minimum and maximum: -0 orders below +0 whatever order
    // the zeros come in, so a group whose least value is zero stores the min
    // -0 when any of its zeros is -0.  (The sign of a zero max never reaches
    // a stored bit: mx - mn is then +0.)
    float mn = v[0], mx = v[0];
    bool finite = true, neg_zero = false, pos_zero = false;
#pragma unroll
    for (int i = 0; i < 64; ++i) {
      finite = finite && __builtin_isfinite(v[i]);
      mn = v[i] < mn ? v[i] : mn;
      mx = v[i] > mx ? v[i] : mx;
      const uint32_t b = __builtin_bit_cast(uint32_t, v[i]);
      neg_zero = neg_zero || b == 0x80000000u;
      pos_zero = pos_zero || b == 0u;
    }
    if (mn == 0.0f) mn = neg_zero ? -0.0f : 0.0f;
    if (mx == 0.0f) mx = pos_zero ? 0.0f : -0.0f;
    const float range = mx - mn;
    const float s32 = range / 15.0f;
    const half_t s16 = (half_t)s32;
    const half_t m16 = (half_t)mn;
    const float sf = (float)s16, mf = (float)m16;
    if (!finite || __builtin_isinf(sf) || __builtin_isinf(mf)) {
      if (err) atomicOr(err, finite ? 2 : 1);
    } else {
      sbits = half_bits(s16);
      mbits = half_bits(m16);
      if (sf != 0.0f) {
#pragma unroll
        for (int i = 0; i < 64; ++i) {
          const float d = v[i] - mf;
          float c = __builtin_rintf(d / sf);
          c = __builtin_fminf(__builtin_fmaxf(c, 0.0f), 15.0f);
          q[i] = (uint8_t)(int)c;
        }
      }
    }
  }
  // Group gamma -> chunk s = gamma / 2, half h = gamma % 2; quarter g holds
  // in-group offsets 16g..16g+15 as two words (8w + c).
  const int s = gamma >> 1, h = gamma & 1;
#pragma unroll
  for (int g = 0; g < 4; ++g) {
    uint32_t wd[2];
#pragma unroll
    for (int wi = 0; wi < 2; ++wi) {
      uint32_t word = 0;
#pragma unroll
      for (int p = 0; p < 8; ++p) word |= (uint32_t)q[16 * g + 8 * wi + kPerm4[p]] << (4 * p);
      wd[wi] = word;
    }
    u32x2 pair = {wd[0], wd[1]};
    *reinterpret_cast<u32x2*>(tile + 1024 * s + 16 * (16 * g + rho) + 8 * h) = pair;
  }
  *reinterpret_cast<uint16_t*>(tile + kMetaOffset4 + 16 * rho + 2 * gamma) = sbits;
  *reinterpret_cast<uint16_t*>(tile + kMetaOffset4 + 16 * rho + 8 + 2 * gamma) = mbits;
}

// One thread per (row-group r, super-block j, block s in 0..7, lane 16g + rho):
// 8 consecutive weights of one row, 16 output bytes.
__global__ __launch_bounds__(256) void pack_fp16_kernel(const float* __restrict__ w, int64_t n,
                                                        int64_t k, uint8_t* __restrict__ out,
                                                        int64_t J, int64_t total,
                                                        int32_t* __restrict__ err) {
  int64_t t = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (t >= total) return;
  const int lane = (int)(t & 63), rho = lane & 15, g = lane >> 4;
  const int s = (int)((t >> 6) & 7);
  const int64_t rj = t >> 9;
  const int64_t j = rj % J;
  const int64_t r = rj / J;
  const int64_t row = r * kTileRows + rho;
  const int64_t k0 = j * kSuperK + 32 * s + 8 * g;
  u32x4 packed = {0u, 0u, 0u, 0u};
  if (row < n && k0 < k) {             // K % 32 == 0: these 8 are wholly in or out
    const float4_t* src = reinterpret_cast<const float4_t*>(w + row * k + k0);
    const float4_t f0 = src[0], f1 = src[1];
    const float v[8] = {f0[0], f0[1], f0[2], f0[3], f1[0], f1[1], f1[2], f1[3]};
    bool finite = true, fits = true;
    uint32_t h[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) {
      finite = finite && __builtin_isfinite(v[i]);
      const half_t hv = (half_t)v[i];
      fits = fits && !__builtin_isinf((float)hv);
      h[i] = half_bits(hv);
    }
    if (!finite || !fits) {
      if (err) atomicOr(err, finite ? 2 : 1);
    } else {
#pragma unroll
      for (int i = 0; i < 4; ++i) packed[i] = h[2 * i] | (h[2 * i + 1] << 16);
    }
  }
  *reinterpret_cast<u32x4*>(out + rj * kTileBytes16 + 1024 * s + 16 * lane) = packed;
}

__global__ void fill_zero_kernel(uint16_t* __restrict__ y, int64_t count) {
  int64_t i = (int64_t)blockIdx.x * blockDim.x + threadIdx.x;
  if (i < count) y[i] = 0;
}

}  // namespace

hipError_t launch_pack_int8(const float* w, int64_t n, int64_t k, uint8_t* out, int32_t* err,
                            hipStream_t s) {
  const int64_t R = ceil_div(n, kTileRows), J = ceil_div(k, kSuperK);
  const int64_t total = R * J * 128;
  if (total == 0) return hipSuccess;
  const int64_t blocks = ceil_div(total, 256);
  hipLaunchKernelGGL(pack_int8_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, w, n, k, out, J,
                     total, err);
  return hipGetLastError();
}

hipError_t launch_pack_int4(const float* w, int64_t n, int64_t k, uint8_t* out, int32_t* err,
                            hipStream_t s) {
  const int64_t R = ceil_div(n, kTileRows), J = ceil_div(k, kSuperK);
  const int64_t total = R * J * 64;
  if (total == 0) return hipSuccess;
  const int64_t blocks = ceil_div(total, 256);
  hipLaunchKernelGGL(pack_int4_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, w, n, k, out, J,
                     total, err);
  return hipGetLastError();
}

hipError_t launch_pack_fp16(const float* w, int64_t n, int64_t k, uint8_t* out, int32_t* err,
                            hipStream_t s) {
  const int64_t R = ceil_div(n, kTileRows), J = ceil_div(k, kSuperK);
  const int64_t total = R * J * 512;
  if (total == 0) return hipSuccess;
  const int64_t blocks = ceil_div(total, 256);
  hipLaunchKernelGGL(pack_fp16_kernel, dim3((uint32_t)blocks), dim3(256), 0, s, w, n, k, out, J,
                     total, err);
  return hipGetLastError();
}

hipError_t launch_fill_zero(uint16_t* y, int64_t count, hipStream_t s) {
  if (count <= 0) return hipSuccess;
  hipLaunchKernelGGL(fill_zero_kernel, dim3((uint32_t)ceil_div(count, 256)), dim3(256), 0, s, y,
                     count);
  return hipGetLastError();
}

}  // namespace qd
