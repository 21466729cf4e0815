// Small-M (1 <= m <= 16) quantized GEMM on the matrix cores: a static chunk of
// up to 16 tokens times an int8 b32 or INT4 g64 weight matrix.  The zoo's Qwen3.8-27B page
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
//
// INT4: a lane holds 16 consecutive codes of its row per 64-wide group (the
// GEMV layout), i.e. two 8-code halves; each half feeds one 16x16x32 MFMA
// whose A operand is the matching 8 activations per lane, so the two MFMAs
// of a group cover its 64 K positions in a permuted order that A and B share.
// Codes become exact fp16 integers (and-or onto 1024, minus 1024).  With
// w^ = min + c s per group, y += s * sum(c x) + min * sum(x): the activation
// sums come from the same two MFMAs run with an all-ones B operand, whose
// every output column is the sum over the group for that token.
//
// Glue: the op's prologue is applied to each A operand as it is loaded (the
// RMSNorm factor of every token is formed once per workgroup first), and its
// epilogue at the store.
#include "glue.h"
#include "qd_internal.h"
#include "tiles.h"

namespace qd {
namespace {

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

// Where a lane's A operands come from: X rows (token m_row), or the two
// blocks of a gated product, or X rows with the token's RMSNorm factor r and
// gamma.  Rows m >= M fall outside the descriptors and read as zeros.
struct ASrc {
  __amdgpu_buffer_rsrc_t rx, rb, rg;
  float r;
};

// Called by every thread of the workgroup (it may hold a barrier).  Under
// RMSNorm, wave w forms the factors of tokens w, w + WAVES, ..., two tokens
// per pass: each lane sums the squares of its 8-value chunks with sixteen
// loads in flight (one memory round trip per two tokens: this runs before the
// workgroup's first product), then the wave adds the lanes' sums in a fixed
// order.
template <int WAVES, int PRO>
__device__ inline ASrc make_asrc(const LinearArgs& a, int m_row, int wave, int lane) {
  const uint32_t xbytes = (uint32_t)(a.m * a.k * 2);
  constexpr bool glu = PRO == QD_PRO_GLU, rms = PRO == QD_PRO_RMSNORM;
  ASrc s;
  s.rx = make_rsrc(a.x, xbytes);
  s.rb = make_rsrc(glu ? a.x + (int64_t)a.m * a.k : a.x, glu ? xbytes : 0u);
  s.rg = make_rsrc(rms ? a.gamma : a.x, rms ? (uint32_t)(a.k * 2) : 0u);
  s.r = 0.0f;
  if constexpr (rms) {
    __shared__ float rinv[QD_MAX_M];
    const int64_t K = a.k;
    for (int t0 = wave; t0 < a.m; t0 += 2 * WAVES) {
      // The second token may be past m: its loads fall outside the buffer
      // (zeros, no traffic) and its factor is not stored.
      const int t1 = t0 + WAVES;
      float ss0 = 0.0f, ss1 = 0.0f;
      for (int64_t i0 = lane * 8; i0 < K; i0 += 512 * 8) {
        u32x4 v0[8], v1[8];
#pragma unroll
        for (int u = 0; u < 8; ++u) {
          v0[u] = bload16(s.rx, (uint32_t)((t0 * K + i0 + 512 * u) * 2));
          v1[u] = bload16(s.rx, (uint32_t)((t1 * K + i0 + 512 * u) * 2));
        }
#pragma unroll
        for (int u = 0; u < 8; ++u)
          if (i0 + 512 * u < K) {
            ss0 = sumsq8(v0[u], ss0);
            ss1 = sumsq8(v1[u], ss1);
          }
      }
      ss0 = wave_sum(ss0);
      ss1 = wave_sum(ss1);
      if (lane == 0) {
        rinv[t0] = rms_inverse(ss0, K, a.eps);
        if (t1 < a.m) rinv[t1] = rms_inverse(ss1, K, a.eps);
      }
    }
    __syncthreads();
    s.r = m_row < a.m ? rinv[m_row] : 0.0f;
  }
  return s;
}

// The 8 multiplied values X'[m_row][kk .. kk + 8) (zero past K).
template <int PRO>
__device__ inline half8_t load_a(const ASrc& s, int64_t K, int m_row, int64_t kk) {
  const uint32_t off = (uint32_t)((m_row * K + kk) * 2);
  u32x4 v = bload16(s.rx, off);
  if constexpr (PRO == QD_PRO_GLU) v = glu8(v, bload16(s.rb, off));
  if constexpr (PRO == QD_PRO_RMSNORM) v = rms8(v, s.r, bload16(s.rg, (uint32_t)(kk * 2)));
  return kk < K ? __builtin_bit_cast(half8_t, v) : (half8_t){};
}

// One workgroup: RG consecutive row-groups (16 weight rows each) x all of K.
// Wave w takes super-blocks j = w, w + WAVES, ...; for each it loads the
// activation block X[0..15][j*256 .. j*256+255] once (8 A operands) and the
// RG weight tiles of that super-block, and issues RG x 8 MFMAs, so each
// activation block read from L2 serves RG tiles.
template <int WAVES, int RG, int TPW, int PRO, bool EPI>
__global__ __launch_bounds__(WAVES * 64) void small_m_int8_kernel(LinearArgs a) {
  __shared__ float4_t red[WAVES][RG][64];
  const int J = a.J;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, rho = lane & 15;
  const uint32_t span = (uint32_t)J * kTileBytes8;
  Owner o[RG];
  __amdgpu_buffer_rsrc_t rw[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    // Row-groups past the launch's last read as zero tiles (empty descriptor)
    // and store nothing.
    const int64_t rg = (int64_t)blockIdx.x * RG + r;
    o[r] = find_owner(a, rg < a.total_rg ? rg : a.total_rg - 1);
    rw[r] = make_rsrc(o[r].blob + o[r].local_rg * (int64_t)span, rg < a.total_rg ? span : 0u);
  }
  const int64_t K = a.k;
  const int m_row = rho;   // A operand row held by this lane
  const ASrc src = make_asrc<WAVES, PRO>(a, m_row, wave, lane);

  float4_t acc[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) acc[r] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = wave; j0 < J; j0 += WAVES * TPW) {
    // Every load of the batch (TPW super-blocks x RG tiles, and their
    // activation blocks) is issued before the first product.  A super-block
    // past K reads zero tiles (no traffic) and zero activations.
    u32x4 c[TPW][RG][4], scw[TPW][RG];
    half8_t xa[TPW][8];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int j = j0 + u * WAVES;
      const uint32_t t = (uint32_t)j * kTileBytes8;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
#pragma unroll
        for (int s = 0; s < 4; ++s) c[u][r][s] = bload16(rw[r], t + 1024 * s + 16 * lane);
        scw[u][r] = bload16(rw[r], t + kMetaOffset8 + 16 * rho);
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int64_t kk = (int64_t)j * kSuperK + 32 * b + 8 * g;
        xa[u][b] = load_a<PRO>(src, K, m_row, kk);
      }
    }
    // Keep every load of the batch ahead of the first product: left alone,
    // the scheduler sinks later tiles' loads to save registers.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const half8_t scales = __builtin_bit_cast(half8_t, scw[u][r]);
#pragma unroll
        for (int s = 0; s < 4; ++s) {
#pragma unroll
          for (int h = 0; h < 2; ++h) {
            const half8_t bq = codes_to_half8(c[u][r][s][2 * h], c[u][r][s][2 * h + 1]);
            const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
            const float4_t p = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[u][2 * s + h], bq, zero, 0, 0, 0);
            const float sc = (float)scales[2 * s + h];
#pragma unroll
            for (int i = 0; i < 4; ++i) acc[r][i] = __builtin_fmaf(sc, p[i], acc[r][i]);
          }
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  // Wave r (< RG) reduces and stores row-group r.
  if (wave < RG) {
    const int r = wave;
    float4_t sum = red[0][r][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const float4_t v = red[w][r][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[i] += v[i];
    }
    const int64_t rg = (int64_t)blockIdx.x * RG + r;
    // Lane (g, rho) holds output rows m = 4g + i of weight row rho.
    Owner ow = o[0];
#pragma unroll
    for (int q = 1; q < RG; ++q)
      if (q == r) ow = o[q];
    const int64_t row = ow.local_rg * kTileRows + rho;
    if (rg < a.total_rg && row < ow.n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < a.m)
          ow.y[(int64_t)m * ow.n + row] =
              EPI ? epilogue_bits(sum[i], ow.epi) : __builtin_bit_cast(uint16_t, (half_t)sum[i]);
      }
    }
  }
}

// fp16 weights (the unquantized head): chunk s of a tile is already the B
// operand of block s; no dequantization and no scale.
template <int WAVES, int RG, int TPW, int PRO, bool EPI>
__global__ __launch_bounds__(WAVES * 64) void small_m_fp16_kernel(LinearArgs a) {
  __shared__ float4_t red[WAVES][RG][64];
  const int J = a.J;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, rho = lane & 15;
  const uint32_t span = (uint32_t)J * kTileBytes16;
  Owner o[RG];
  __amdgpu_buffer_rsrc_t rw[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t rg = (int64_t)blockIdx.x * RG + r;
    o[r] = find_owner(a, rg < a.total_rg ? rg : a.total_rg - 1);
    rw[r] = make_rsrc(o[r].blob + o[r].local_rg * (int64_t)span, rg < a.total_rg ? span : 0u);
  }
  const int64_t K = a.k;
  const int m_row = rho;
  const ASrc src = make_asrc<WAVES, PRO>(a, m_row, wave, lane);

  float4_t acc[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) acc[r] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = wave; j0 < J; j0 += WAVES * TPW) {
    u32x4 c[TPW][RG][8];
    half8_t xa[TPW][8];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int j = j0 + u * WAVES;
      const uint32_t t = (uint32_t)j * kTileBytes16;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
#pragma unroll
        for (int s = 0; s < 8; ++s) c[u][r][s] = bload16(rw[r], t + 1024 * s + 16 * lane);
      }
#pragma unroll
      for (int b = 0; b < 8; ++b) {
        const int64_t kk = (int64_t)j * kSuperK + 32 * b + 8 * g;
        xa[u][b] = load_a<PRO>(src, K, m_row, kk);
      }
    }
    // Keep every load of the batch ahead of the first product: left alone,
    // the scheduler sinks later tiles' loads to save registers.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
#pragma unroll
      for (int r = 0; r < RG; ++r) {
#pragma unroll
        for (int b = 0; b < 8; ++b)
          acc[r] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[u][b], __builtin_bit_cast(half8_t, c[u][r][b]),
                                                          acc[r], 0, 0, 0);
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave < RG) {
    const int r = wave;
    float4_t sum = red[0][r][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const float4_t v = red[w][r][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[i] += v[i];
    }
    const int64_t rg = (int64_t)blockIdx.x * RG + r;
    Owner ow = o[0];
#pragma unroll
    for (int q = 1; q < RG; ++q)
      if (q == r) ow = o[q];
    const int64_t row = ow.local_rg * kTileRows + rho;
    if (rg < a.total_rg && row < ow.n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < a.m)
          ow.y[(int64_t)m * ow.n + row] =
              EPI ? epilogue_bits(sum[i], ow.epi) : __builtin_bit_cast(uint16_t, (half_t)sum[i]);
      }
    }
  }
}

// INT4 g64: one workgroup = RG row-groups x all of K, waves along K (as above).
template <int WAVES, int RG, int TPW, int PRO, bool EPI>
__global__ __launch_bounds__(WAVES * 64) void small_m_int4_kernel(LinearArgs a) {
  __shared__ float4_t red[WAVES][RG][64];
  const int J = a.J;
  const int lane = threadIdx.x & 63, wave = threadIdx.x >> 6, g = lane >> 4, rho = lane & 15;
  const uint32_t span = (uint32_t)J * kTileBytes4;
  Owner o[RG];
  __amdgpu_buffer_rsrc_t rw[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) {
    const int64_t rg = (int64_t)blockIdx.x * RG + r;
    o[r] = find_owner(a, rg < a.total_rg ? rg : a.total_rg - 1);
    rw[r] = make_rsrc(o[r].blob + o[r].local_rg * (int64_t)span, rg < a.total_rg ? span : 0u);
  }
  const int64_t K = a.k;
  const int m_row = rho;
  const ASrc src = make_asrc<WAVES, PRO>(a, m_row, wave, lane);
  const half_t one = (half_t)1.0f;
  const half8_t ones = {one, one, one, one, one, one, one, one};
  const half2_t minus1024 = {(half_t)-1024.0f, (half_t)-1024.0f};

  float4_t acc[RG];
#pragma unroll
  for (int r = 0; r < RG; ++r) acc[r] = (float4_t){0.0f, 0.0f, 0.0f, 0.0f};
  for (int j0 = wave; j0 < J; j0 += WAVES * TPW) {
    u32x4 c[TPW][RG][2], meta[TPW][RG];
    half8_t xa[TPW][8];
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      const int j = j0 + u * WAVES;
      const uint32_t t = (uint32_t)j * kTileBytes4;
#pragma unroll
      for (int r = 0; r < RG; ++r) {
#pragma unroll
        for (int s = 0; s < 2; ++s) c[u][r][s] = bload16(rw[r], t + 1024 * s + 16 * lane);
        meta[u][r] = bload16(rw[r], t + kMetaOffset4 + 16 * rho);
      }
      // A operands: group gam, half h -> X[m][j*256 + 64 gam + 16 g + 8 h .. +8].
#pragma unroll
      for (int q = 0; q < 8; ++q) {
        const int64_t kk = (int64_t)j * kSuperK + 64 * (q >> 1) + 16 * g + 8 * (q & 1);
        xa[u][q] = load_a<PRO>(src, K, m_row, kk);
      }
    }
    // Keep every load of the batch ahead of the first product: left alone,
    // the scheduler sinks later tiles' loads to save registers.
    __builtin_amdgcn_sched_barrier(0);
#pragma unroll
    for (int u = 0; u < TPW; ++u) {
      // Per group: sum of x over its 64 positions, for this lane's tokens.
      float4_t xs[4];
#pragma unroll
      for (int gam = 0; gam < 4; ++gam) {
        const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
        xs[gam] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[u][2 * gam], ones, zero, 0, 0, 0);
        xs[gam] = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[u][2 * gam + 1], ones, xs[gam], 0, 0, 0);
      }
#pragma unroll
      for (int r = 0; r < RG; ++r) {
        const half8_t mt = __builtin_bit_cast(half8_t, meta[u][r]);
#pragma unroll
        for (int gam = 0; gam < 4; ++gam) {
          const int s = gam >> 1, h = gam & 1;
          float4_t pc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
          for (int half = 0; half < 2; ++half) {
            // 8 codes (k order) of this lane's row: nibble p holds code (0,2,4,6,1,3,5,7)[p].
            const uint32_t wd = c[u][r][s][2 * h + half];
            const uint32_t mk = 0x000F000Fu, e = 0x64006400u;
            const half2_t c01 = as_h2((wd & mk) | e) + minus1024;
            const half2_t c23 = as_h2(((wd >> 4) & mk) | e) + minus1024;
            const half2_t c45 = as_h2(((wd >> 8) & mk) | e) + minus1024;
            const half2_t c67 = as_h2(((wd >> 12) & mk) | e) + minus1024;
            const half8_t bq = {c01[0], c01[1], c23[0], c23[1], c45[0], c45[1], c67[0], c67[1]};
            pc = __builtin_amdgcn_mfma_f32_16x16x32_f16(xa[u][2 * gam + half], bq, pc, 0, 0, 0);
          }
          const float sc = (float)mt[gam], mn = (float)mt[4 + gam];
#pragma unroll
          for (int i = 0; i < 4; ++i)
            acc[r][i] = __builtin_fmaf(sc, pc[i], __builtin_fmaf(mn, xs[gam][i], acc[r][i]));
        }
      }
    }
  }
#pragma unroll
  for (int r = 0; r < RG; ++r) red[wave][r][lane] = acc[r];
  __syncthreads();
  if (wave < RG) {
    const int r = wave;
    float4_t sum = red[0][r][lane];
#pragma unroll
    for (int w = 1; w < WAVES; ++w) {
      const float4_t v = red[w][r][lane];
#pragma unroll
      for (int i = 0; i < 4; ++i) sum[i] += v[i];
    }
    const int64_t rg = (int64_t)blockIdx.x * RG + r;
    Owner ow = o[0];
#pragma unroll
    for (int q = 1; q < RG; ++q)
      if (q == r) ow = o[q];
    const int64_t row = ow.local_rg * kTileRows + rho;
    if (rg < a.total_rg && row < ow.n) {
#pragma unroll
      for (int i = 0; i < 4; ++i) {
        const int m = 4 * g + i;
        if (m < a.m)
          ow.y[(int64_t)m * ow.n + row] =
              EPI ? epilogue_bits(sum[i], ow.epi) : __builtin_bit_cast(uint16_t, (half_t)sum[i]);
      }
    }
  }
}

template <int W, int RG, int TPW, int PRO, bool EPI>
void launch_cfg(int fmt, dim3 grid, const LinearArgs& a, hipStream_t s) {
  if (fmt == QD_FMT_INT4_G64)
    hipLaunchKernelGGL((small_m_int4_kernel<W, RG, TPW, PRO, EPI>), grid, dim3(W * 64), 0, s, a);
  else if (fmt == QD_FMT_FP16)
    hipLaunchKernelGGL((small_m_fp16_kernel<W, RG, TPW, PRO, EPI>), grid, dim3(W * 64), 0, s, a);
  else
    hipLaunchKernelGGL((small_m_int8_kernel<W, RG, TPW, PRO, EPI>), grid, dim3(W * 64), 0, s, a);
}

// Launch shapes, chosen by a sweep over the Qwen3 2B/4B/8B and 27B-shaped
// projections at m = 16 on MI355X (each shape's launches back to back):
//  * many row-groups (gate|up, the head): 4-wave workgroups of 2 row-groups
//    (below 2048 row-groups) or 4 row-groups (more), so each activation block
//    serves 2 or 4 tiles and several workgroups stay resident per CU;
//  * fewer (q|k|v, o, down: one or two per CU): one row-group per workgroup;
//    int8 waves issue two super-blocks' loads before their first product
//    (4 waves), INT4 and fp16 waves one (8 waves).
enum SmallShape { kRg4W4 = 0, kRg2W4 = 1, kW4T2 = 2, kW8T1 = 3, kW4T1 = 4 };

int pick_small_m(int fmt, int64_t total_rg, int J) {
  // INT4 tiles are half the bytes of int8 ones: four row-groups per
  // workgroup already from 1024 (8B INT4 M=16 step 2048 vs 2068 us).
  if (fmt == QD_FMT_INT4_G64 && total_rg >= 4 * 256 && J >= 8) return kRg4W4;
  if (total_rg >= 4 * 256 && J >= 8) return total_rg >= 2048 ? kRg4W4 : kRg2W4;
  if (J < 8) return kW4T1;
  return fmt == QD_FMT_INT8_B32 ? kW4T2 : kW8T1;
}

template <int PRO, bool EPI>
hipError_t launch_small_m_pro(int fmt, const LinearArgs& a, hipStream_t s, int shape) {
  if (fmt != QD_FMT_INT4_G64 && fmt != QD_FMT_FP16 && fmt != QD_FMT_INT8_B32) return hipErrorInvalidValue;
  const dim3 grid1((uint32_t)a.total_rg);
  switch (shape) {
    case kRg4W4: launch_cfg<4, 4, 1, PRO, EPI>(fmt, dim3((uint32_t)ceil_div(a.total_rg, 4)), a, s); break;
    case kRg2W4: launch_cfg<4, 2, 1, PRO, EPI>(fmt, dim3((uint32_t)ceil_div(a.total_rg, 2)), a, s); break;
    case kW4T2: launch_cfg<4, 1, 2, PRO, EPI>(fmt, grid1, a, s); break;
    case kW8T1: launch_cfg<8, 1, 1, PRO, EPI>(fmt, grid1, a, s); break;
    default: launch_cfg<4, 1, 1, PRO, EPI>(fmt, grid1, a, s); break;
  }
  return hipGetLastError();
}

}  // namespace

// The prologue and the presence of an epilogue are template parameters: the
// kernels without glue are the plain ones, with nothing of the glue in them.
hipError_t launch_small_m(int fmt, const LinearArgs& a, hipStream_t s) {
  if (a.total_rg == 0) return hipSuccess;
  const bool epi = has_glue(a);     // any epilogue (or prologue): the storing kernels
  int shape = pick_small_m(fmt, a.total_rg, a.J);
  // RMSNorm-fed groups of a few hundred row-groups: two per workgroup, so
  // each workgroup's per-token statistic serves two row-groups (glued 8B
  // M=16 step 3481 vs 3526 us; the gated product is better with one: 4110).
  if (a.pro == QD_PRO_RMSNORM && a.J >= 8 && a.total_rg < 4 * 256) shape = kRg2W4;
  switch (a.pro) {
    case QD_PRO_RMSNORM: return launch_small_m_pro<QD_PRO_RMSNORM, true>(fmt, a, s, shape);
    case QD_PRO_GLU: return launch_small_m_pro<QD_PRO_GLU, true>(fmt, a, s, shape);
    default:
      return epi ? launch_small_m_pro<QD_PRO_NONE, true>(fmt, a, s, shape)
                 : launch_small_m_pro<QD_PRO_NONE, false>(fmt, a, s, shape);
  }
}

}  // namespace qd
