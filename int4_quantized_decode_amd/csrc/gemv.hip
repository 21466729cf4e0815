// M = 1 quantized GEMV kernels (one decoded token).
//
// The pages put decode time in streaming the quantized weights once per token
// (Qwen3-VL 4B/8B Core AI cards, Measured paragraph: "Decode is
// bandwidth-bound").  These kernels are shaped for that stream on CDNA4:
//   * one workgroup per row-group of 16 rows; its waves stride over the 256-K
//     super-blocks, so every wave load is one contiguous 1 KiB (64 lanes x
//     16 B) of the tiled blob, and every packed byte is read exactly once;
//   * weight loads are raw buffer loads whose descriptor spans one row-group,
//     so the next tile can be requested unconditionally: a request past the
//     row-group returns zeros without touching memory;
//   * the activation vector is staged once per workgroup in LDS (zero-padded
//     to the super-block), read back by quarter-lane groups;
//   * dequantization happens in registers: int8 codes become exact fp16 values
//     through a byte permute onto the fp16 pattern of 1024 (+128 bias) and one
//     packed subtraction; int4 codes through an and-or onto 1024, with the
//     bias folded into the group's min term.  Products run on v_dot2 with
//     fp32 accumulation; the block scale is applied once per 8 codes;
//   * per-row partial sums are reduced across the 4 lanes of a row with lane
//     shuffles, then across waves through LDS, and rounded once to fp16.
#include "qd_internal.h"

namespace qd {
namespace {

constexpr int kDescWord3 = 0x00020000;   // raw buffer, gfx9-family data format

__device__ inline __amdgpu_buffer_rsrc_t make_rsrc(const void* base, uint32_t bytes) {
  return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, kDescWord3);
}

__device__ inline u32x4 bload16(__amdgpu_buffer_rsrc_t r, uint32_t off) {
  return __builtin_amdgcn_raw_buffer_load_b128(r, off, 0, 0);
}

__device__ inline half2_t as_h2(uint32_t v) { return __builtin_bit_cast(half2_t, v); }

// sum_{i<8} q_i x_i for 8 int8 codes in (d0, d1) (k order) and 8 fp16 x.
// Each code byte b is biased to b ^ 0x80 = q + 128 and permuted under the
// fp16 exponent byte 0x64, giving the exact fp16 value 1024 + 128 + q; one
// packed subtraction of 1152 leaves q exactly.
__device__ inline float dot8_int8(uint32_t d0, uint32_t d1, half8_t x, float acc) {
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

// sum_{i<8} (1024 + c_i) x_i for one int4 word (nibble p holds code
// k0 + (0,2,4,6,1,3,5,7)[p]), so each and-or yields the pair (k0+2t, k0+2t+1).
__device__ inline float dot8_int4_biased(uint32_t w, half8_t x, float acc) {
  const uint32_t m = 0x000F000Fu, e = 0x64006400u;
  const half2_t c01 = as_h2((w & m) | e);
  const half2_t c23 = as_h2(((w >> 4) & m) | e);
  const half2_t c45 = as_h2(((w >> 8) & m) | e);
  const half2_t c67 = as_h2(((w >> 12) & m) | e);
  acc = __builtin_amdgcn_fdot2(c01, (half2_t){x[0], x[1]}, acc, false);
  acc = __builtin_amdgcn_fdot2(c23, (half2_t){x[2], x[3]}, acc, false);
  acc = __builtin_amdgcn_fdot2(c45, (half2_t){x[4], x[5]}, acc, false);
  acc = __builtin_amdgcn_fdot2(c67, (half2_t){x[6], x[7]}, acc, false);
  return acc;
}

struct Tile8 {
  u32x4 c[4];
  u32x4 sc;
};

struct Tile4 {
  u32x4 c[2];
  u32x4 meta;
};

__device__ inline Tile8 load_tile8(__amdgpu_buffer_rsrc_t r, int j, int lane) {
  const uint32_t t = (uint32_t)j * kTileBytes8;
  Tile8 T;
#pragma unroll
  for (int s = 0; s < 4; ++s) T.c[s] = bload16(r, t + 1024 * s + 16 * lane);
  T.sc = bload16(r, t + kMetaOffset8 + 16 * (lane & 15));
  return T;
}

__device__ inline Tile4 load_tile4(__amdgpu_buffer_rsrc_t r, int j, int lane) {
  const uint32_t t = (uint32_t)j * kTileBytes4;
  Tile4 T;
#pragma unroll
  for (int s = 0; s < 2; ++s) T.c[s] = bload16(r, t + 1024 * s + 16 * lane);
  T.meta = bload16(r, t + kMetaOffset4 + 16 * (lane & 15));
  return T;
}

// Lane (g, rho)'s share of one int8 tile: row rho, K quarter g, 8 blocks.
__device__ inline float tile_dot8(const Tile8& T, const half_t* xs_j, int g, float acc) {
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
// y += s * sum (1024 + c) x + (m - 1024 s) * sum x  ==  sum (m + c s) x.
__device__ inline float tile_dot4(const Tile4& T, const half_t* xs_j, const float* xsum_j, int g,
                                  float acc) {
  const half8_t meta = __builtin_bit_cast(half8_t, T.meta);
  const float4_t xsum = *reinterpret_cast<const float4_t*>(xsum_j + 4 * g);
#pragma unroll
  for (int s = 0; s < 2; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const int gam = 2 * s + h;
      const half_t* xp = xs_j + 64 * gam + 16 * g;
      const half8_t xa = *reinterpret_cast<const half8_t*>(xp);
      const half8_t xb = *reinterpret_cast<const half8_t*>(xp + 8);
      float p = dot8_int4_biased(T.c[s][2 * h], xa, 0.0f);
      p = dot8_int4_biased(T.c[s][2 * h + 1], xb, p);
      const float sc = (float)meta[gam], mn = (float)meta[4 + gam];
      acc = __builtin_fmaf(sc, p, acc);
      acc = __builtin_fmaf(__builtin_fmaf(-1024.0f, sc, mn), xsum[gam], acc);
    }
  }
  return acc;
}

// Resolve which member matrix owns row-group `rg` (selects, no indexing).
struct Owner {
  const uint8_t* blob;
  uint16_t* y;
  int64_t n;
  int64_t local_rg;
};

__device__ inline Owner find_owner(const LinearArgs& a, int64_t rg) {
  Owner o{a.mem[0].blob, a.mem[0].y, a.mem[0].n, rg};
#pragma unroll
  for (int i = 1; i < kMaxMembers; ++i) {
    if (i < a.n_mem && rg >= a.mem[i].rg_begin) {
      o.blob = a.mem[i].blob;
      o.y = a.mem[i].y;
      o.n = a.mem[i].n;
      o.local_rg = rg - a.mem[i].rg_begin;
    }
  }
  return o;
}

// Stage x (fp16 [k], zero beyond k) into LDS, 16 bytes per thread per step.
template <int THREADS>
__device__ inline void stage_x(const LinearArgs& a, half_t* xs) {
  const int Kp = a.J * kSuperK;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(a.k * 2));
  for (int i = threadIdx.x * 8; i < Kp; i += THREADS * 8)
    *reinterpret_cast<u32x4*>(xs + i) = bload16(rx, (uint32_t)i * 2);
}

// Each wave owns super-blocks j = wave + t * WAVES, t < TPW, of one row-group,
// and WAVES * TPW >= J.  All of a wave's tile loads are issued in straight-line
// code before any of them is consumed; a tile past the row-group reads as
// zeros (no traffic) and contributes nothing, so no branch guards a load.
template <int WAVES, int TPW>
__global__ __launch_bounds__(WAVES * 64) void gemv_int8_kernel(LinearArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int J = a.J;
  half_t* xs = reinterpret_cast<half_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)J * kSuperK * 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;

  const Owner o = find_owner(a, blockIdx.x);
  const uint32_t span = (uint32_t)J * kTileBytes8;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(o.blob + o.local_rg * (int64_t)span, span);

  Tile8 T[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) T[t] = load_tile8(rw, wave + t * WAVES, lane);
  stage_x<WAVES * 64>(a, xs);
  __syncthreads();

  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int j = min(wave + t * WAVES, J - 1);   // x of a zero tile: any valid run
    acc = tile_dot8(T[t], xs + j * kSuperK, g, acc);
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w * 16 + lane];
    const int64_t row = o.local_rg * kTileRows + lane;
    if (row < o.n) o.y[row] = __builtin_bit_cast(uint16_t, (half_t)sum);
  }
}

template <int WAVES, int TPW>
__global__ __launch_bounds__(WAVES * 64) void gemv_int4_kernel(LinearArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int J = a.J;
  half_t* xs = reinterpret_cast<half_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + (size_t)J * kSuperK * 2);   // [J][g][gamma]
  float* red = xsum + (size_t)J * 16;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;

  const Owner o = find_owner(a, blockIdx.x);
  const uint32_t span = (uint32_t)J * kTileBytes4;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(o.blob + o.local_rg * (int64_t)span, span);

  Tile4 T[TPW];
#pragma unroll
  for (int t = 0; t < TPW; ++t) T[t] = load_tile4(rw, wave + t * WAVES, lane);
  stage_x<WAVES * 64>(a, xs);
  __syncthreads();
  // Sum of each 16-value run of x at k = 256j + 64 gamma + 16 g, stored at
  // index 16 j + 4 g + gamma.
  for (int t = threadIdx.x; t < J * 16; t += WAVES * 64) {
    const half8_t v0 = *reinterpret_cast<const half8_t*>(xs + 16 * t);
    const half8_t v1 = *reinterpret_cast<const half8_t*>(xs + 16 * t + 8);
    float sum = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += (float)v0[i];
#pragma unroll
    for (int i = 0; i < 8; ++i) sum += (float)v1[i];
    const int jj = t >> 4, within = t & 15;
    xsum[16 * jj + 4 * (within & 3) + (within >> 2)] = sum;
  }
  __syncthreads();

  float acc = 0.0f;
#pragma unroll
  for (int t = 0; t < TPW; ++t) {
    const int j = min(wave + t * WAVES, J - 1);
    acc = tile_dot4(T[t], xs + j * kSuperK, xsum + 16 * j, g, acc);
  }
  acc += __shfl_xor(acc, 16);
  acc += __shfl_xor(acc, 32);
  if (lane < 16) red[wave * 16 + lane] = acc;
  __syncthreads();
  if (wave == 0 && lane < 16) {
    float sum = 0.0f;
#pragma unroll
    for (int w = 0; w < WAVES; ++w) sum += red[w * 16 + lane];
    const int64_t row = o.local_rg * kTileRows + lane;
    if (row < o.n) o.y[row] = __builtin_bit_cast(uint16_t, (half_t)sum);
  }
}

constexpr int kMaxTPW = 6;

void pick_shape(int64_t total_rg, int J, int* waves, int* tpw) {
  int w = 16;
  while (w > 4 && (w > J || total_rg * w > 256 * 32)) w /= 2;
  int t = (J + w - 1) / w;
  if (t > kMaxTPW) {
    w = 16;
    t = (J + w - 1) / w;
  }
  *waves = w;
  *tpw = t;
}

template <int W, int TPW>
void launch_one(int fmt, const LinearArgs& a, hipStream_t s, size_t lds) {
  const dim3 grid((uint32_t)a.total_rg), block(W * 64);
  if (fmt == QD_FMT_INT8_B32) hipLaunchKernelGGL((gemv_int8_kernel<W, TPW>), grid, block, lds, s, a);
  else hipLaunchKernelGGL((gemv_int4_kernel<W, TPW>), grid, block, lds, s, a);
}

template <int W>
void launch_w(int fmt, int tpw, const LinearArgs& a, hipStream_t s, size_t lds) {
  switch (tpw) {
    case 1: launch_one<W, 1>(fmt, a, s, lds); break;
    case 2: launch_one<W, 2>(fmt, a, s, lds); break;
    case 3: launch_one<W, 3>(fmt, a, s, lds); break;
    case 4: launch_one<W, 4>(fmt, a, s, lds); break;
    case 5: launch_one<W, 5>(fmt, a, s, lds); break;
    default: launch_one<W, 6>(fmt, a, s, lds); break;
  }
}

}  // namespace

hipError_t launch_gemv(int fmt, const LinearArgs& a, hipStream_t s) {
  if (a.total_rg == 0) return hipSuccess;
  int W, TPW;
  pick_shape(a.total_rg, a.J, &W, &TPW);
  size_t lds = (size_t)a.J * kSuperK * 2 + (size_t)W * 16 * 4;
  if (fmt == QD_FMT_INT4_G64) lds += (size_t)a.J * 16 * 4;
  if (W == 16) launch_w<16>(fmt, TPW, a, s, lds);
  else if (W == 8) launch_w<8>(fmt, TPW, a, s, lds);
  else launch_w<4>(fmt, TPW, a, s, lds);
  return hipGetLastError();
}

}  // namespace qd
