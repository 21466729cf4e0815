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
//     shuffles, then across waves through LDS, and rounded once to fp16;
//   * the op's prologue (RMSNorm, gated product) is applied while x is staged
//     and its epilogue (silu) at the store, so the glue costs no pass of its
//     own.
#include "glue.h"
#include "qd_internal.h"
#include "tiles.h"

namespace qd {
namespace {

// Resolve which member matrix owns row-group `rg` (selects, no indexing).
struct Owner {
  const uint8_t* blob;
  uint16_t* y;
  int64_t n;
  int64_t local_rg;
  int epi;
};

__device__ inline Owner find_owner(const LinearArgs& a, int64_t rg) {
  Owner o{a.mem[0].blob, a.mem[0].y, a.mem[0].n, rg, a.mem[0].epi};
#pragma unroll
  for (int i = 1; i < kMaxMembers; ++i) {
    if (i < a.n_mem && rg >= a.mem[i].rg_begin) {
      o.blob = a.mem[i].blob;
      o.y = a.mem[i].y;
      o.n = a.mem[i].n;
      o.local_rg = rg - a.mem[i].rg_begin;
      o.epi = a.mem[i].epi;
    }
  }
  return o;
}

// Stage the multiplied vector (fp16 [k], zero beyond k) into LDS, 16 bytes per
// thread per step, applying the prologue.  Under RMSNorm the raw x goes to
// xs and gamma to `aux` (J * 256 halves) in the same pass; after one barrier
// every thread forms the statistic from the per-wave sums in the same order
// and normalises its own chunks.  The caller's barrier follows.
template <int THREADS, bool GLUE>
__device__ inline void stage_x(const LinearArgs& a, half_t* xs, half_t* aux) {
  const int Kp = a.J * kSuperK;
  const uint32_t xbytes = (uint32_t)(a.k * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, xbytes);
  if (!GLUE || a.pro == QD_PRO_NONE) {
    for (int i = threadIdx.x * 8; i < Kp; i += THREADS * 8)
      *reinterpret_cast<u32x4*>(xs + i) = bload16(rx, (uint32_t)i * 2);
    return;
  }
  if (a.pro == QD_PRO_GLU) {
    const __amdgpu_buffer_rsrc_t rb = make_rsrc(a.x + a.k, xbytes);   // one token: B follows A
    for (int i = threadIdx.x * 8; i < Kp; i += THREADS * 8)
      *reinterpret_cast<u32x4*>(xs + i) = glu8(bload16(rx, (uint32_t)i * 2), bload16(rb, (uint32_t)i * 2));
    return;
  }
  __shared__ float wsum[THREADS / 64];
  const __amdgpu_buffer_rsrc_t rg = make_rsrc(a.gamma, xbytes);
  float ss = 0.0f;
  for (int i = threadIdx.x * 8; i < Kp; i += THREADS * 8) {
    const u32x4 v = bload16(rx, (uint32_t)i * 2);
    *reinterpret_cast<u32x4*>(aux + i) = bload16(rg, (uint32_t)i * 2);
    *reinterpret_cast<u32x4*>(xs + i) = v;
    ss = sumsq8(v, ss);
  }
  ss = wave_sum(ss);
  if ((threadIdx.x & 63) == 0) wsum[threadIdx.x >> 6] = ss;
  __syncthreads();
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < THREADS / 64; ++w) tot += wsum[w];
  const float r = rms_inverse(tot, a.k, a.eps);
  for (int i = threadIdx.x * 8; i < Kp; i += THREADS * 8)
    *reinterpret_cast<u32x4*>(xs + i) =
        rms8(*reinterpret_cast<const u32x4*>(xs + i), r, *reinterpret_cast<const u32x4*>(aux + i));
}

// Each wave owns super-blocks j = wave + t * WAVES, t < TPW, of one row-group,
// and WAVES * TPW >= J.  All of a wave's tile loads are issued in straight-line
// code before any of them is consumed; a tile past the row-group reads as
// zeros (no traffic) and contributes nothing, so no branch guards a load.
template <int WAVES, int TPW, bool GLUE>
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
  stage_x<WAVES * 64, GLUE>(a, xs, reinterpret_cast<half_t*>(red + WAVES * 16));
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
    if (row < o.n) o.y[row] = GLUE ? epilogue_bits(sum, o.epi) : __builtin_bit_cast(uint16_t, (half_t)sum);
  }
}

template <int WAVES, int TPW, bool GLUE>
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
  stage_x<WAVES * 64, GLUE>(a, xs, reinterpret_cast<half_t*>(red + WAVES * 16));
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
    if (row < o.n) o.y[row] = GLUE ? epilogue_bits(sum, o.epi) : __builtin_bit_cast(uint16_t, (half_t)sum);
  }
}

// fp16 tiles are twice as large as int8 ones: at most kBatch16 of them are held
// in registers at once; a wave with more tiles loads the next batch after
// computing the previous one.
constexpr int kBatch16 = 3;

template <int WAVES, int TPW, bool GLUE>
__global__ __launch_bounds__(WAVES * 64) void gemv_fp16_kernel(LinearArgs a) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  const int J = a.J;
  half_t* xs = reinterpret_cast<half_t*>(smem);
  float* red = reinterpret_cast<float*>(smem + (size_t)J * kSuperK * 2);
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4;

  const Owner o = find_owner(a, blockIdx.x);
  const uint32_t span = (uint32_t)J * kTileBytes16;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(o.blob + o.local_rg * (int64_t)span, span);

  constexpr int B = TPW < kBatch16 ? TPW : kBatch16;
  Tile16 T[B];
#pragma unroll
  for (int t = 0; t < B; ++t) T[t] = load_tile16(rw, wave + t * WAVES, lane);
  stage_x<WAVES * 64, GLUE>(a, xs, reinterpret_cast<half_t*>(red + WAVES * 16));
  __syncthreads();

  float acc = 0.0f;
#pragma unroll
  for (int t0 = 0; t0 < TPW; t0 += B) {
    if (t0 > 0) {
#pragma unroll
      for (int t = 0; t < B; ++t)
        if (t0 + t < TPW) T[t] = load_tile16(rw, wave + (t0 + t) * WAVES, lane);
    }
#pragma unroll
    for (int t = 0; t < B; ++t) {
      if (t0 + t < TPW) {
        const int j = min(wave + (t0 + t) * WAVES, J - 1);
        acc = tile_dot16(T[t], xs + j * kSuperK, g, acc);
      }
    }
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
    if (row < o.n) o.y[row] = GLUE ? epilogue_bits(sum, o.epi) : __builtin_bit_cast(uint16_t, (half_t)sum);
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

// GLUE selects the kernels that apply a prologue or epilogue; the others are
// the plain ones, with nothing of the glue in them.
template <int W, int TPW>
void launch_one(int fmt, const LinearArgs& a, hipStream_t s, size_t lds) {
  const dim3 grid((uint32_t)a.total_rg), block(W * 64);
  if (has_glue(a)) {
    if (fmt == QD_FMT_INT8_B32) hipLaunchKernelGGL((gemv_int8_kernel<W, TPW, true>), grid, block, lds, s, a);
    else if (fmt == QD_FMT_INT4_G64) hipLaunchKernelGGL((gemv_int4_kernel<W, TPW, true>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((gemv_fp16_kernel<W, TPW, true>), grid, block, lds, s, a);
  } else {
    if (fmt == QD_FMT_INT8_B32) hipLaunchKernelGGL((gemv_int8_kernel<W, TPW, false>), grid, block, lds, s, a);
    else if (fmt == QD_FMT_INT4_G64) hipLaunchKernelGGL((gemv_int4_kernel<W, TPW, false>), grid, block, lds, s, a);
    else hipLaunchKernelGGL((gemv_fp16_kernel<W, TPW, false>), grid, block, lds, s, a);
  }
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
  if (a.pro == QD_PRO_RMSNORM) lds += (size_t)a.J * kSuperK * 2;   // gamma
  if (W == 16) launch_w<16>(fmt, TPW, a, s, lds);
  else if (W == 8) launch_w<8>(fmt, TPW, a, s, lds);
  else launch_w<4>(fmt, TPW, a, s, lds);
  return hipGetLastError();
}

}  // namespace qd
