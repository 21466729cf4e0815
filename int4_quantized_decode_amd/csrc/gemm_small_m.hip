// Small-M (1 <= m <= 16) quantized GEMM on the matrix cores: a static chunk of
// up to 16 tokens times an int8 b32 weight matrix.  The zoo's Qwen3.8-27B page
// (vision path section) runs prefill as static S=16 chunks beside the S=1
// decode function; this is that contraction.
//
// Mapping: one v_mfma_f32_16x16x32_f16 per (16 rows, one 32-wide block).  The
// tiled layout already gives each lane the operand it needs: lane l = 16g +
// rho holds 8 codes of weight row rho at K offsets 8g..8g+7 of a block, which
// is the B operand (K x N, N = weight row) of the 16x16x32 instruction, and
// the A operand is X[m = l % 16][same 8 K offsets].  Codes become exact fp16
// (the same permute as the GEMV), each block's product is scaled by that
// block's fp16 scale in fp32, and the 16 x 16 fp32 results are reduced across
// waves in LDS.  The path stays bound by the weight stream: at m = 16 each
// weight byte feeds 32 flops.
#include "qd_internal.h"
#include "tiles.h"

namespace qd {
namespace {

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

template <int WAVES>
__global__ __launch_bounds__(WAVES * 64) void small_m_int8_kernel(LinearArgs a) {
  __shared__ float4_t red[WAVES][64];
  const int J = a.J;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, rho = lane & 15;
  const Owner o = find_owner(a, blockIdx.x);
  const uint32_t span = (uint32_t)J * kTileBytes8;
  const __amdgpu_buffer_rsrc_t rw = make_rsrc(o.blob + o.local_rg * (int64_t)span, span);
  // X rows m >= M fall outside the descriptor and read as zeros.
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(a.x, (uint32_t)(a.m * a.k * 2));
  const int64_t K = a.k;
  const int m_row = rho;   // A operand row held by this lane

  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int j = wave; j < J; j += WAVES) {
    const uint32_t t = (uint32_t)j * kTileBytes8;
    u32x4 c[4];
#pragma unroll
    for (int s = 0; s < 4; ++s) c[s] = bload16(rw, t + 1024 * s + 16 * lane);
    const u32x4 scw = bload16(rw, t + kMetaOffset8 + 16 * rho);
    half8_t xa[8];
#pragma unroll
    for (int b = 0; b < 8; ++b) {
      const int64_t kk = (int64_t)j * kSuperK + 32 * b + 8 * g;
      const u32x4 v = bload16(rx, (uint32_t)((m_row * K + kk) * 2));
      xa[b] = kk < K ? __builtin_bit_cast(half8_t, v) : (half8_t){};
    }
    const half8_t scales = __builtin_bit_cast(half8_t, scw);
#pragma unroll
    for (int s = 0; s < 4; ++s) {
#pragma unroll
      for (int h = 0; h < 2; ++h) {
        const half8_t bq = codes_to_half8(c[s][2 * h], c[s][2 * h + 1]);
        const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
        const float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[2 * s + h], bq, zero, 0, 0, 0);
        const float sc = (float)scales[2 * s + h];
#pragma unroll
        for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, p[i], acc[i]);
      }
    }
  }
  red[wave][lane] = acc;
  __syncthreads();
  if (wave == 0) {
    float4_t sum = red[0][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const float4_t v = red[w][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[i] += v[i];
    }
    // Lane (g, rho) holds output rows m = 4g + i of weight row rho.
    const int64_t row = o.local_rg * kTileRows + rho;
    if (row < o.n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < a.m) o.y[(int64_t)m * o.n + row] = __builtin_bit_cast(uint16_t, (half_t)sum[i]);
      }
    }
  }
}

}  // namespace

hipError_t launch_small_m(int fmt, const LinearArgs& a, hipStream_t s) {
  if (a.total_rg == 0) return hipSuccess;
  if (fmt != QD_FMT_INT8_B32) return hipErrorInvalidValue;
  const dim3 grid((uint32_t)a.total_rg);
  int w = 16;
  while (w > 4 && (w > a.J || a.total_rg * w > 256 * 32)) w /= 2;
  if (w == 16) hipLaunchKernelGGL(small_m_int8_kernel<16>, grid, dim3(16 * 64), 0, s, a);
  else if (w == 8) hipLaunchKernelGGL(small_m_int8_kernel<8>, grid, dim3(8 * 64), 0, s, a);
  else hipLaunchKernelGGL(small_m_int8_kernel<4>, grid, dim3(4 * 64), 0, s, a);
  return hipGetLastError();
}

}  // namespace qd
