// Internal declarations shared by the HIP translation units of libqdecode.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

#include "../../include/qdecode.h"

namespace qd {

// Tiled-layout constants (see the layout description in qdecode.h).
constexpr int kTileRows = 16;
constexpr int kSuperK = 256;
constexpr int kTileBytes8 = 4352;   // 4 x 1024 code bytes + 256 scale bytes
constexpr int kTileBytes4 = 2304;   // 2 x 1024 code bytes + 256 scale/min bytes
constexpr int kTileBytes16 = 8192;  // 8 x 1024 bytes of fp16 weights (unquantized head)
constexpr int kMetaOffset8 = 4096;
constexpr int kMetaOffset4 = 2048;

typedef _Float16 half_t;
typedef half_t half2_t __attribute__((ext_vector_type(2)));
typedef half_t half4_t __attribute__((ext_vector_type(4)));
typedef half_t half8_t __attribute__((ext_vector_type(8)));
typedef float float4_t __attribute__((ext_vector_type(4)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

inline int64_t ceil_div(int64_t a, int64_t b) { return (a + b - 1) / b; }

inline int tile_bytes(int fmt) {
  return fmt == QD_FMT_INT8_B32 ? kTileBytes8 : fmt == QD_FMT_INT4_G64 ? kTileBytes4 : kTileBytes16;
}

// Up to this many matrices share one activation vector in a fused launch.
constexpr int kMaxMembers = 4;

struct Member {
  const uint8_t* blob;   // tiled blob of this matrix
  uint16_t* y;           // output, [m, n] fp16 bits
  int64_t n;             // rows of this matrix
  int64_t rg_begin;      // first row-group of this member in the launch's index space
  int32_t epi;           // qd_epilogue applied to this member's outputs
};

struct LinearArgs {
  Member mem[kMaxMembers];
  int n_mem;
  int J;                 // super-blocks per row (Kp / 256)
  int64_t k;             // logical K
  int64_t total_rg;      // sum of row-groups over members
  const uint16_t* x;     // [m, k] fp16 bits ([2, m, k] under QD_PRO_GLU)
  int m;                 // token rows (1..16)
  int pro;               // qd_prologue applied to x
  const uint16_t* gamma; // QD_PRO_RMSNORM weight, fp16 [k]
  float eps;             // QD_PRO_RMSNORM epsilon
};

// Whether a launch applies any glue (a prologue, or an epilogue on a member).
inline bool has_glue(const LinearArgs& a) {
  bool g = a.pro != QD_PRO_NONE;
  for (int i = 0; i < a.n_mem; ++i) g = g || a.mem[i].epi != QD_EPI_NONE;
  return g;
}

// Launchers (enqueue only; arguments already validated).
hipError_t launch_pack_int8(const float* w, int64_t n, int64_t k, uint8_t* out, int32_t* err,
                            hipStream_t s);
hipError_t launch_pack_int4(const float* w, int64_t n, int64_t k, uint8_t* out, int32_t* err,
                            hipStream_t s);
hipError_t launch_pack_fp16(const float* w, int64_t n, int64_t k, uint8_t* out, int32_t* err,
                            hipStream_t s);
hipError_t launch_gemv(int fmt, const LinearArgs& a, hipStream_t s);
hipError_t launch_small_m(int fmt, const LinearArgs& a, hipStream_t s);
hipError_t launch_fill_zero(uint16_t* y, int64_t count, hipStream_t s);
hipError_t launch_read_probe(const void* buf, uint64_t bytes, uint32_t* sink, int grid, hipStream_t s);

}  // namespace qd
