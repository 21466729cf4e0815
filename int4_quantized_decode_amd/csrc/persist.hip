// Persistent decode-step kernel: one launch walks every group of the step.
//
// Decode streams every quantized weight once per token (Qwen3-VL 4B/8B Core
// AI cards, Measured paragraph), so a step's time is the weight stream plus
// whatever stalls it.  Per-group launches stall it at every group boundary:
// the next kernel starts loading only after the previous one drains.  Here the
// weight stream keeps going across group boundaries:
//
//   * one workgroup per CU (cooperative launch, all co-resident), 16 waves:
//     streaming compute waves, reserve compute waves and 1 control wave.  The
//     workgroup's share of every group's schedule lives in LDS, so no wave
//     waits on a memory round trip to find its next tiles;
//   * a group's row-groups are split into one contiguous range per
//     workgroup; compute waves take tiles (at up to 16 token rows: units of
//     two row-groups at one super-block) of the workgroup's sequence from an
//     LDS counter, in order, across group boundaries;
//   * a streaming wave keeps a ring of tiles in registers and refills a slot
//     as soon as it is consumed.  Its loads are accepted only as fast as
//     memory delivers, so at a group boundary its ring holds landed data and
//     it has nothing more to issue; reserve waves hold no tiles until the
//     workgroup has computed every tile of a group and then issue the next
//     tiles while the device synchronises, so memory keeps streaming;
//   * compute waves write each tile's partials to their own LDS slot and
//     count the tile against its row-group; the control wave reduces and
//     stores each row-group as soon as it is complete (fixed-order sums:
//     deterministic), publishes that the workgroup has finished the group
//     (one completion stamp per workgroup), waits until every workgroup has
//     published it, and releases the compute waves (one barrier per group),
//     so an op may consume an earlier op's output;
//   * one token row: the control wave stages each group's activation vector
//     (and, with glue, gamma or the gated product's second block) straight
//     into LDS and applies the prologue there;
//   * up to 16 token rows: compute waves read the activation blocks
//     themselves, from copies in matrix-core order where the plan keeps them
//     (made before the step, or written by the op producing them), and the
//     partials are 16 x 16 per tile; groups too large for the partials in
//     LDS are split into row ranges that need no device-wide wait between
//     them;
//   * compute waves issue no global stores or atomics.
//
// Ordering around each boundary is decided from the step's buffers when the
// plan is made: activations no earlier group writes are read ahead of the
// barrier with ordinary loads; outputs a later group reads or rewrites are
// acknowledged before the stamp; activations an earlier group wrote are read
// after it, device-coherently unless no cache can hold a stale copy of their
// lines.  Outputs and stamps are written with device-coherent stores.  No
// L2-wide write-back or invalidate is issued.
//
// Waits are bounded: a wait that exceeds its spin limit sets an error word
// and every later wait is skipped, so the kernel always finishes.
#include <algorithm>
#include <cstring>
#include <map>
#include <new>
#include <vector>

#include "glue.h"
#include "stack.h"
#include "tiles.h"

namespace qd {

namespace {

constexpr int kWaves = 16;
constexpr int kCtl = 15;                // the control wave
// Compute waves are waves 0 .. 14: the first kCtl - R stream continuously,
// the last R (a kernel template parameter, chosen per format and row count
// from measurements; see kernel_ptr) load only while the workgroup stalls.
constexpr uint32_t kSpinLimit = 1u << 20;   // default wait bound, polls (each a device-coherent
                                            // round trip): ~1 s; a plan may set another

// Ordering a group needs around its boundary, from the plan's overlap
// analysis of the step's buffers.
enum : int32_t {
  kStageEarly = 1,      // no earlier group writes any byte of x: it may be staged before the barrier
  kAckOutputs = 2,      // a later group reads or rewrites an output: stores complete before the stamp
  kNoWait = 4,          // a further row range of the op(s) before: no device-wide wait at the boundary
  kCleanLines = 8,      // x is written earlier in the step, but no cache can hold a stale copy of its
                        // lines: after the barrier it is read through the caches
};

struct PGroup {         // 64 bytes
  const uint16_t* x;
  const uint16_t* gamma;  // RMSNorm weight (prologue QD_PRO_RMSNORM)
  const uint16_t* xt;     // m > 1: x in matrix-core order (plan scratch), or null
  int64_t k;
  int32_t J;            // super-blocks per row
  int32_t R;            // row-groups in the group
  int32_t mem0;         // first member in the member table
  int32_t n_mem;
  int32_t pro;          // qd_prologue of the group's input
  float eps;
  int32_t order;        // kStageEarly | kAckOutputs | kNoWait | kCleanLines
  int32_t pad;
};

struct PMember {        // 48 bytes
  const uint8_t* blob;
  uint16_t* y;
  int64_t n;
  int32_t rg_begin;     // first row-group of this member within its group
  int32_t epi;          // qd_epilogue of this member's outputs
  int64_t ld;           // elements between token rows of y (m > 1)
  uint16_t* yt;         // m > 1: where the outputs also go in matrix-core order, or null
};

struct PSched {         // 16 bytes: one workgroup's part of one group
  int32_t n;            // tiles (whole row-groups: a multiple of the group's J)
  int32_t off;          // tiles of this workgroup in the groups before this one
  int32_t rg0;          // first row-group
  int32_t nseg;         // row-groups (rg0, rg0 + 1, ...)
};

static_assert(sizeof(PGroup) % 16 == 0 && sizeof(PMember) % 16 == 0 && sizeof(PSched) == 16,
              "schedule records are copied to LDS in 16-byte units");

struct PlanArgs {
  const PGroup* groups;       // [ngroups]
  const PMember* members;     // [nmem]
  const PSched* sched;        // [ngroups][G]
  unsigned long long* flags;  // [G] completion stamps
  uint32_t* err;
  unsigned long long epoch;   // runs so far, including this one
  int32_t ngroups;
  int32_t nmem;
  int32_t G;
  int32_t x_bytes;            // LDS layout: x (+ second operand) | xsum | red | cnt | groups | members | sched
  int32_t xsum_bytes;
  int32_t red_bytes;
  int32_t cnt_bytes;
  int32_t tab_bytes;
  int32_t m;                  // token rows (1 .. 16)
  uint32_t spin_limit;        // bound of every wait, in polls
};

template <int FMT> struct Fmt;
template <> struct Fmt<QD_FMT_INT8_B32> {
  using Tile = Tile8;
  static constexpr int kT = kTileBytes8;
  __device__ static Tile load(__amdgpu_buffer_rsrc_t r, int lane) { return load_tile8(r, 0, lane); }
};
template <> struct Fmt<QD_FMT_INT4_G64> {
  using Tile = Tile4;
  static constexpr int kT = kTileBytes4;
  __device__ static Tile load(__amdgpu_buffer_rsrc_t r, int lane) { return load_tile4(r, 0, lane); }
};

__device__ __forceinline__ void wg_barrier() {
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  __builtin_amdgcn_s_barrier();
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

__device__ __forceinline__ int uni(int v) { return __builtin_amdgcn_readfirstlane(v); }

// Flags and counters other waves of the workgroup update, in LDS.  Relaxed
// workgroup-scope atomics compile to plain LDS reads and writes; a volatile
// access through a generic pointer would become a flat access, which also
// counts against the wave's vector-memory counter and so waits for the
// wave's weight loads in flight.
template <typename T>
__device__ __forceinline__ T lds_get(const T* p) {
  return __hip_atomic_load(p, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}
template <typename T>
__device__ __forceinline__ void lds_put(T* p, T v) {
  __hip_atomic_store(p, v, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
}

template <typename T>
__device__ __forceinline__ T* uni_ptr(T* ptr) {
  const uint64_t u = reinterpret_cast<uint64_t>(ptr);
  const uint32_t lo = (uint32_t)uni((int)(uint32_t)u), hi = (uint32_t)uni((int)(uint32_t)(u >> 32));
  return reinterpret_cast<T*>(((uint64_t)hi << 32) | lo);
}

// The workgroup's schedule, resident in LDS.  Reads are wave-uniform.
struct Sched {
  const PGroup* g;
  const PMember* m;
  const PSched* s;
  __device__ int J(int gi) const { return uni(g[gi].J); }
  __device__ int R(int gi) const { return uni(g[gi].R); }
  __device__ int mem0(int gi) const { return uni(g[gi].mem0); }
  __device__ int nmem(int gi) const { return uni(g[gi].n_mem); }
  __device__ const uint16_t* x(int gi) const { return uni_ptr(g[gi].x); }
  __device__ const uint16_t* gamma(int gi) const { return uni_ptr(g[gi].gamma); }
  __device__ const uint16_t* xt(int gi) const { return uni_ptr(g[gi].xt); }
  __device__ int pro(int gi) const { return uni(g[gi].pro); }
  __device__ int order(int gi) const { return uni(g[gi].order); }
  __device__ float eps(int gi) const { return __builtin_bit_cast(float, uni(__builtin_bit_cast(int, g[gi].eps))); }
  __device__ int64_t k(int gi) const { return (int64_t)uni((int)g[gi].k); }
  __device__ int tiles(int gi) const { return uni(s[gi].n); }
  __device__ int off(int gi) const { return uni(s[gi].off); }
  __device__ int rg0(int gi) const { return uni(s[gi].rg0); }
  __device__ int nseg(int gi) const { return uni(s[gi].nseg); }
  __device__ int rg_begin(int mi) const { return uni(m[mi].rg_begin); }
  __device__ const uint8_t* blob(int mi) const { return uni_ptr(m[mi].blob); }
  __device__ uint16_t* y(int mi) const { return uni_ptr(m[mi].y); }
  __device__ int64_t n(int mi) const { return (int64_t)uni((int)m[mi].n); }
  // Per-lane reads, for a member index that may differ between lanes.
  __device__ int rg_begin_l(int mi) const { return m[mi].rg_begin; }
  __device__ uint16_t* y_l(int mi) const { return m[mi].y; }
  __device__ int64_t n_l(int mi) const { return m[mi].n; }
  __device__ int epi_l(int mi) const { return m[mi].epi; }
  __device__ int64_t ld(int mi) const { return (int64_t)uni((int)m[mi].ld); }
  __device__ uint16_t* yt(int mi) const { return uni_ptr(m[mi].yt); }
};

// Tile hand-out.  A workgroup's tiles of all groups form one sequence
// (group by group, row-group major); compute waves take the next index from
// an LDS counter whenever a ring slot frees.  Tiles are therefore fetched in
// sequence order whatever the waves' relative progress, so a group completes
// when its last tile lands, and loads for the next groups queue behind it.
struct TileRef {
  int g;      // group (ngroups: no tile)
  int j;      // super-block within the row
  int rel;    // partial slot: the tile's index in the workgroup's range of the group
              // (row-group major; a unit's: its first tile's)
  int seg;    // row-group within the range (a unit's: its first)
  int nv;     // units: row-groups the unit holds
};

struct IssueCursor {
  int g;                // current group (-1 before the first)
  int off_next;         // sequence index where the next group starts
  int u, seg, j;        // last issued tile (or unit): index within the workgroup's part,
                        // (segment, super-block); for units seg counts units
  int J, rg0, nseg;
  int mem, mem_last;
};

template <int FMT>
__device__ __forceinline__ typename Fmt<FMT>::Tile issue(const Sched& S, int ngroups, int total,
                                                         uint32_t* next, IssueCursor& c,
                                                         TileRef& ref, int lane, bool take = true) {
  constexpr int T = Fmt<FMT>::kT;
  // take == false: claim nothing; the load below then reads an empty buffer
  // (zeros, no memory traffic), which keeps the caller's control flow uniform.
  uint32_t got = (uint32_t)total;
  if (take && lane == 0) got = atomicAdd(next, 1u);
  const int idx = uni((int)got);
  const uint8_t* base = nullptr;
  uint32_t nbytes = 0;
  ref.g = ngroups;
  if (idx < total) {
    while (idx >= c.off_next) {                       // enter the group holding idx
      ++c.g;
      c.J = S.J(c.g);
      c.rg0 = S.rg0(c.g);
      c.nseg = S.nseg(c.g);
      c.off_next = c.g + 1 < ngroups ? S.off(c.g + 1) : total;
      c.u = 0;
      c.seg = 0;
      c.j = 0;
      c.mem = S.mem0(c.g);
      c.mem_last = c.mem + S.nmem(c.g) - 1;
    }
    const int u = idx - S.off(c.g);
    c.j += u - c.u;
    c.u = u;
    while (c.j >= c.J) {
      c.j -= c.J;
      ++c.seg;
    }
    const int rg = c.rg0 + c.seg;
    while (c.mem < c.mem_last && rg >= S.rg_begin(c.mem + 1)) ++c.mem;
    base = S.blob(c.mem) + ((int64_t)(rg - S.rg_begin(c.mem)) * c.J + c.j) * T;
    nbytes = T;
    ref.g = c.g;
    ref.j = c.j;
    ref.rel = u;
    ref.seg = c.seg;
  }
  return Fmt<FMT>::load(make_rsrc(base, nbytes), lane);
}

// Up to 16 token rows: the sequence is made of units, U row-groups at one
// super-block (unit-row major: units (q, 0), (q, 1), ... (q, J - 1), then
// q + 1), so that one activation block serves U tiles.  The last unit of a
// range may hold fewer row-groups; its missing tiles read as zeros.
template <int FMT, int U>
struct Unit {
  typename Fmt<FMT>::Tile w[U];
};

template <int FMT, int U>
__device__ __forceinline__ Unit<FMT, U> issue_unit(const Sched& S, int ngroups, int total, uint32_t* next,
                                                   IssueCursor& c, TileRef& ref, int lane, bool take = true) {
  constexpr int T = Fmt<FMT>::kT;
  uint32_t got = (uint32_t)total;
  if (take && lane == 0) got = atomicAdd(next, 1u);
  const int idx = uni((int)got);
  const uint8_t* base[U];
  uint32_t nbytes[U];
#pragma unroll
  for (int q = 0; q < U; ++q) {
    base[q] = nullptr;
    nbytes[q] = 0;
  }
  ref.g = ngroups;
  ref.nv = 0;
  if (idx < total) {
    while (idx >= c.off_next) {                       // enter the group holding idx
      ++c.g;
      c.J = S.J(c.g);
      c.rg0 = S.rg0(c.g);
      c.nseg = S.nseg(c.g);
      c.off_next = c.g + 1 < ngroups ? S.off(c.g + 1) : total;
      c.u = 0;
      c.seg = 0;
      c.j = 0;
      c.mem = S.mem0(c.g);
      c.mem_last = c.mem + S.nmem(c.g) - 1;
    }
    const int u = idx - S.off(c.g);
    c.j += u - c.u;
    c.u = u;
    while (c.j >= c.J) {                              // c.seg counts units here
      c.j -= c.J;
      ++c.seg;
    }
    const int seg0 = c.seg * U;
    const int nv = min(U, c.nseg - seg0);
    // The cursor follows the member of the unit's first row-group, which
    // only moves forward along the sequence.  A unit's later row-groups may
    // lie in the next members: each finds its own from there, without
    // moving the cursor, since the unit's next super-block starts again
    // from its first row-group.
    while (c.mem < c.mem_last && c.rg0 + seg0 >= S.rg_begin(c.mem + 1)) ++c.mem;
#pragma unroll
    for (int q = 0; q < U; ++q) {
      if (q < nv) {
        const int rg = c.rg0 + seg0 + q;
        int mi = c.mem;
        while (mi < c.mem_last && rg >= S.rg_begin(mi + 1)) ++mi;
        base[q] = S.blob(mi) + ((int64_t)(rg - S.rg_begin(mi)) * c.J + c.j) * T;
        nbytes[q] = T;
      }
    }
    ref.g = c.g;
    ref.j = c.j;
    ref.rel = seg0 * c.J + c.j;                       // partial slot of the unit's first tile
    ref.seg = seg0;
    ref.nv = nv;
  }
  Unit<FMT, U> t;
#pragma unroll
  for (int q = 0; q < U; ++q) t.w[q] = Fmt<FMT>::load(make_rsrc(base[q], nbytes[q]), lane);
  return t;
}

// Reserve-wave pacing, in ticks of the 100 MHz real-time counter per tile:
// kT / 256 ticks per tile is 25.6 GB/s per CU, about one CU's share of the
// HBM bandwidth; QD_PLAN_PACE_PCT scales that rate.
#ifndef QD_PLAN_PACE_PCT
#define QD_PLAN_PACE_PCT 100
#endif
template <int FMT>
__device__ __forceinline__ uint32_t pace_ticks(int k) {
  return (uint32_t)(((int64_t)k * Fmt<FMT>::kT * 100) / (256 * QD_PLAN_PACE_PCT));
}

template <int FMT>
__device__ __forceinline__ float tile_dot(const typename Fmt<FMT>::Tile& T, const half_t* xs,
                                          const float* xsum, int j, int g, float acc);
template <>
__device__ __forceinline__ float tile_dot<QD_FMT_INT8_B32>(const Tile8& T, const half_t* xs,
                                                           const float*, int j, int g, float acc) {
  return tile_dot8(T, xs + j * kSuperK, g, acc);
}
template <>
__device__ __forceinline__ float tile_dot<QD_FMT_INT4_G64>(const Tile4& T, const half_t* xs,
                                                           const float* xsum, int j, int g, float acc) {
  return tile_dot4(T, xs + j * kSuperK, xsum + 16 * j, g, acc);
}

// Up to 16 token rows (MT = 16).  The activation block of super-block j,
// X[0..15][256 j .. 256 j + 255], as the eight A operands of the tile's
// 16x16x32 products: operand q of lane (gq, rho) holds token rho's 8 values
// at K position kpos(q, gq) within the super-block:
//   int8 b32: 32 q + 8 gq                       (operand q = 32-block q)
//   INT4 g64: 64 (q / 2) + 16 gq + 8 (q % 2)    (operands 2a, 2a + 1 = group a;
//                                                the lane's 16 consecutive codes)
template <int FMT>
__host__ __device__ constexpr int kpos(int q, int gq) {
  return FMT == QD_FMT_INT8_B32 ? 32 * q + 8 * gq : 64 * (q >> 1) + 16 * gq + 8 * (q & 1);
}

// The blocks are read from memory, not staged (16 x K does not fit in LDS for
// the longest K).
//
// Matrix-core order: where the plan keeps a copy of x in it (xt), 16-byte
// chunk (8 j + q) 64 + lane holds operand q of super-block j for that lane
// (zeros past m and past K), so each operand load is one contiguous KiB.
// Copies are written only where nothing can leave a stale line of them in a
// cache, and are read through the caches.
//
// Otherwise x is read in place: token rows past m and K positions past K read
// as zeros (out-of-range offsets: no memory traffic).  Activations nothing in
// the step writes go through the caches; the others are read
// device-coherently unless their lines are known clean.
template <int FMT>
__device__ __forceinline__ void load_xblock(const Sched& S, int g, int j, int m, int lane,
                                            bool coherent, u32x4 (&xa)[8]) {
  const uint16_t* xt = S.xt(g);
  if (xt) {
    const __amdgpu_buffer_rsrc_t rt = make_rsrc(xt, (uint32_t)S.J(g) * 8192u);
#pragma unroll
    for (int b = 0; b < 8; ++b) xa[b] = bload16(rt, (uint32_t)((j * 8 + b) * 1024 + lane * 16));
    return;
  }
  const int gq = lane >> 4, rho = lane & 15;
  const int64_t K = S.k(g);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(S.x(g), (uint32_t)(m * K * 2));
#pragma unroll
  for (int b = 0; b < 8; ++b) {
    const int64_t kk = (int64_t)j * kSuperK + kpos<FMT>(b, gq);
    const uint32_t off = kk < K ? (uint32_t)((rho * K + kk) * 2) : 0x80000000u;
    xa[b] = coherent ? bload16_coherent(rx, off) : bload16(rx, off);
  }
}

// Where output row n (of a K-long input row of a later group) goes in that
// group's matrix-core-ordered copy, token row t: the inverse of kpos.
template <int FMT>
__device__ __forceinline__ int64_t xt_index(int64_t n, int t) {
  const int64_t j = n >> 8;
  const int w = (int)(n & 255);
  const int q = FMT == QD_FMT_INT8_B32 ? w >> 5 : 2 * (w >> 6) + ((w >> 3) & 1);
  const int gq = FMT == QD_FMT_INT8_B32 ? (w >> 3) & 3 : (w >> 4) & 3;
  return (((j * 8 + q) * 64 + gq * 16 + t) << 3) + (w & 7);
}

// The tile's 16 x 16 product with the activation block on the matrix cores
// (B operand = the lane's 8 codes of one 32-block, as in the small-M
// kernels).  Lane (gq, rho) gets tokens 4 gq + i of weight row rho.
__device__ __forceinline__ float4_t tile_mfma(const Tile8& T, const u32x4 (&xa)[8], const float4_t*) {
  const half8_t scales = __builtin_bit_cast(half8_t, T.sc);
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const half8_t bq = codes_to_half8(T.c[s][2 * h], T.c[s][2 * h + 1]);
      const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
      const float4_t pr = __builtin_amdgcn_mfma_f32_16x16x32_f16(
          __builtin_bit_cast(half8_t, xa[2 * s + h]), bq, zero, 0, 0, 0);
      const float sc = (float)scales[2 * s + h];
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, pr[i], acc[i]);
    }
  }
  return acc;
}

// INT4 g64, per group a: codes as exact fp16 integers (nibble p of a word
// holds code (0,2,4,6,1,3,5,7)[p]) through two MFMAs, then
// y += scale * sum(c x) + min * sum(x), the group's activation sums coming
// from the same operands against an all-ones B (group_sums, once per unit).
__device__ __forceinline__ void group_sums(const u32x4 (&xa)[8], float4_t (&xs)[4]) {
  const half_t one = (half_t)1.0f;
  const half8_t ones = {one, one, one, one, one, one, one, one};
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
    xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, xa[2 * a]), ones, zero, 0, 0, 0);
    xs[a] = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, xa[2 * a + 1]), ones, xs[a], 0, 0, 0);
  }
}

__device__ __forceinline__ float4_t tile_mfma(const Tile4& T, const u32x4 (&xa)[8], const float4_t* xs) {
  const half8_t mt = __builtin_bit_cast(half8_t, T.meta);
  const half2_t minus1024 = {(half_t)-1024.0f, (half_t)-1024.0f};
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int s = a >> 1, h = a & 1;
    float4_t pc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
    for (int half = 0; half < 2; ++half) {
      const uint32_t wd = T.c[s][2 * h + half];
      const uint32_t mk = 0x000F000Fu, e = 0x64006400u;
      const half2_t c01 = as_h2((wd & mk) | e) + minus1024;
      const half2_t c23 = as_h2(((wd >> 4) & mk) | e) + minus1024;
      const half2_t c45 = as_h2(((wd >> 8) & mk) | e) + minus1024;
      const half2_t c67 = as_h2(((wd >> 12) & mk) | e) + minus1024;
      const half8_t bq = {c01[0], c01[1], c23[0], c23[1], c45[0], c45[1], c67[0], c67[1]};
      pc = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, xa[2 * a + half]), bq, pc, 0, 0, 0);
    }
    const float sc = (float)mt[a], mn = (float)mt[4 + a];
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] = __builtin_fmaf(sc, pc[i], __builtin_fmaf(mn, xs[a][i], acc[i]));
  }
  return acc;
}

// Keep a load where it is written: the scheduler may not move code across
// the barrier, and the memory clobber stops earlier passes from sinking the
// load towards its first use (which would empty the ring).
#define QD_PIN_ISSUE()                  \
  do {                                  \
    __builtin_amdgcn_sched_barrier(0);  \
    asm volatile("" ::: "memory");      \
  } while (0)

// Compute waves come in two kinds.
//
// A streaming wave keeps a ring of D tiles and refills a slot as soon as it is
// consumed, following the workgroup's tile sequence across group boundaries.
// Its loads are accepted by the memory pipeline only as fast as memory
// delivers, so when the workgroup stalls at a group boundary (the next
// group's activations need every workgroup to finish), its ring already holds
// landed data and it has nothing more to issue: on its own the weight stream
// would idle for the length of the stall.
//
// A reserve wave holds no tiles while the stream runs.  When the workgroup has
// computed every tile of a group (the control wave says so through `stalled`),
// it takes the next S tiles of the sequence and issues them, so memory keeps
// streaming while the workgroup synchronises; it computes them once their
// group's activations are staged, then waits for the next stall.
//
// Both wait for "activations of group g staged" (one workgroup barrier per
// group).  After each tile a wave writes the tile's partials (16 row sums;
// 16 x 16 at up to 16 token rows) to their own LDS slot and counts the tile
// against its row-group, so the control wave can finish a row-group as soon
// as its last tile is in.
template <int FMT, int MT, int U> struct RingOf { using type = typename Fmt<FMT>::Tile; };
template <int FMT, int U> struct RingOf<FMT, 16, U> { using type = Unit<FMT, U>; };

template <int FMT, int D, bool RESERVE, int R, int MT, int U>
__device__ void compute_wave(const PlanArgs& p, const Sched& S, int total, uint32_t* next,
                             int lane, const half_t* xs, const float* xsum, float* red,
                             uint32_t* cnt, const int* stalled, const int* staged) {
  using Tile = typename RingOf<FMT, MT, U>::type;
  const int ng = p.ngroups;
  const int g4 = lane >> 4;
  IssueCursor ic{-1, 0, 0, 0, 0, 1, 0, 0, 0, 0};
  Tile ring[D];
  TileRef ref[D];
  auto next_tile = [&](TileRef& r, int ln, bool take = true) {
    if constexpr (MT == 1) return issue<FMT>(S, ng, total, next, ic, r, ln, take);
    else return issue_unit<FMT, U>(S, ng, total, next, ic, r, ln, take);
  };
  // MT > 1: each slot's activation block, loaded with the tile when the
  // block is already readable (nothing in the step writes it, or its group's
  // boundary has passed), else when the tile is computed.
  u32x4 xr[MT > 1 ? D : 1][8];
  bool xl[MT > 1 ? D : 1];
  int cg = -1;                      // last group whose activations this wave has waited for
  auto settle_to = [&](int g) {
    while (cg < g) {
      ++cg;
      if (cg < ng) wg_barrier();
    }
  };
  auto early_x = [&](int s) {
    if constexpr (MT > 1) {
      xl[s] = false;
      if (ref[s].g < ng) {
        const int ord = S.order(ref[s].g);
        const bool early = (ord & kStageEarly) != 0;
        if (early || uni(lds_get(staged)) >= ref[s].g) {
          load_xblock<FMT>(S, ref[s].g, ref[s].j, p.m, lane, !(ord & (kStageEarly | kCleanLines)), xr[s]);
          xl[s] = true;
        }
      }
    }
  };
  auto compute = [&](int s) {
    const Tile& t = ring[s];
    const TileRef& r = ref[s];
    settle_to(r.g);
    if constexpr (MT == 1) {
      const float part = quad_reduce(tile_dot<FMT>(t, xs, xsum, r.j, g4, 0.0f));
      if (lane < 16) red[r.rel * 16 + lane] = part;
    } else {
      if (!xl[s]) load_xblock<FMT>(S, r.g, r.j, p.m, lane, !(S.order(r.g) & (kStageEarly | kCleanLines)), xr[s]);
      // Each tile's 16 x 16 partial, one float4 per lane, in the tile's own
      // slot (row-group seg + q: J slots further on).
      const int J = S.J(r.g);
      float4_t xs4[4];
      if constexpr (FMT == QD_FMT_INT4_G64) group_sums(xr[s], xs4);
#pragma unroll
      for (int q = 0; q < U; ++q)
        if (q < r.nv) reinterpret_cast<float4_t*>(red)[(r.rel + q * J) * 64 + lane] = tile_mfma(t.w[q], xr[s], xs4);
    }
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) {
      if constexpr (MT == 1) {
        __hip_atomic_fetch_add(cnt + r.seg, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      } else {
#pragma unroll
        for (int q = 0; q < U; ++q)
          if (q < r.nv)
            __hip_atomic_fetch_add(cnt + r.seg + q, 1u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
      }
    }
  };
  if (!RESERVE) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      ring[s] = next_tile(ref[s], lane);
      early_x(s);
      QD_PIN_ISSUE();
    }
    // The ring is consumed and refilled in slot order with a single loop
    // exit, so each compute waits only for its own slot's loads.
    for (;;) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        if (ref[s].g < ng) compute(s);
        ring[s] = next_tile(ref[s], lane);
        early_x(s);
        QD_PIN_ISSUE();
      }
      if (ref[0].g >= ng) break;   // slot 0 was refilled first: nothing left for later slots
    }
  } else {
    const int r = uni((int)(threadIdx.x >> 6)) - (kCtl - R);   // rank among reserve waves
    int trig = 0;                   // issue at the stall that ends group `trig`
    for (;;) {
      // Pass the barrier of group `trig` first: the control wave reaches the
      // next barrier only after the stall of `trig`, so this wait holds up
      // no barrier.
      settle_to(trig);
      // Wait for the stall that ends group `trig` (or, should it have been
      // missed, for the next activations: then nothing is issued).
      for (uint32_t spins = 0;
           lds_get(stalled) < trig && lds_get(staged) <= trig && spins < p.spin_limit; ++spins)
        __builtin_amdgcn_s_sleep(1);
      // Issue at a bounded rate rather than all at once (the control wave's
      // stores and loads on the boundary's critical path queue behind what
      // the CU has in flight), and only while the stall lasts: once the next
      // activations are staged the streaming waves are loading again.
      const uint32_t t0 = (uint32_t)__builtin_amdgcn_s_memrealtime();
      bool stop = false, exhausted = false;
#pragma unroll
      for (int s = 0; s < D; ++s) {
        const uint32_t due = t0 + pace_ticks<FMT>((s * R + r) * (MT == 1 ? 1 : U));
        while (!stop && (int32_t)((uint32_t)__builtin_amdgcn_s_memrealtime() - due) < 0) {
          stop = lds_get(staged) > trig;
          if (!stop) __builtin_amdgcn_s_sleep(2);
        }
        stop = stop || lds_get(staged) > trig;
        ring[s] = next_tile(ref[s], lane, !stop);
        early_x(s);
        exhausted = exhausted || (!stop && ref[s].g >= ng);
        QD_PIN_ISSUE();
      }
#pragma unroll
      for (int s = 0; s < D; ++s)
        if (ref[s].g < ng) compute(s);
      if (exhausted) break;         // the sequence is used up
      trig = cg > trig ? cg : trig + 1;
    }
  }
  settle_to(ng);
}

// ---- control wave ----------------------------------------------------------

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ unsigned long long stamp(const PlanArgs& p, int g) {
  return p.epoch * (unsigned long long)p.ngroups + (unsigned long long)(g + 1);
}

// Move Kp halves from `r` into LDS at xs, 64 lanes x 16 bytes per load,
// straight from memory (no registers); past the descriptor the loads read
// zeros.  Each load fills 512 halves, so the LDS written is Kp rounded up to
// a multiple of 512 halves (x_span).  The caller waits.
__host__ __device__ constexpr int x_span(int Kp) { return (Kp + 511) / 512 * 512; }

template <int POLICY>
__device__ __forceinline__ void dma_to_lds(__amdgpu_buffer_rsrc_t r, int Kp, int lane, half_t* xs) {
  for (int i = 0; i < Kp; i += 512)
    __builtin_amdgcn_raw_ptr_buffer_load_lds(
        r, (__attribute__((address_space(3))) void*)(xs + i), 16, (uint32_t)(i * 2 + lane * 16), 0,
        0, POLICY);
}

// Stage a group's multiplied vector (and, for int4, its 16-value run sums) in
// LDS.  All loads, and under a prologue the second operand's (gamma, or the
// gated product's B block) into xs + x_span(Kp), are issued before the single wait,
// so staging costs one memory round trip whatever K is.  The prologue then
// runs in place: each lane rewrites the 8-value chunks its own loads brought.
// POLICY: device-coherent for activations an earlier group of the step may
// have written (unless no cache can hold a stale copy of their lines); cached
// for the others, so the workgroups of an XCD share one L2 copy (8B step
// 1367-1372 vs 1375-1378 us coherent).
template <int FMT, bool GLUE, int POLICY = kPolicyCoherent>
__device__ __forceinline__ void stage_group_x(const Sched& S, int g, int lane, half_t* xs,
                                              float* xsum) {
  const int Kp = S.J(g) * kSuperK;
  const int64_t k = S.k(g);
  const uint32_t xbytes = (uint32_t)(k * 2);
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(S.x(g), xbytes);
  dma_to_lds<POLICY>(rx, Kp, lane, xs);
  if constexpr (GLUE) {
    const int pro = S.pro(g);
    half_t* const xs2 = xs + x_span(Kp);            // second operand, after x's whole span
    if (pro == QD_PRO_GLU) dma_to_lds<POLICY>(make_rsrc(S.x(g) + k, xbytes), Kp, lane, xs2);
    if (pro == QD_PRO_RMSNORM) dma_to_lds<POLICY>(make_rsrc(S.gamma(g), xbytes), Kp, lane, xs2);
    wait_stores();                                 // vmcnt(0): the data is in LDS
    if (pro == QD_PRO_GLU) {
      for (int i = lane * 8; i < Kp; i += 512)
        *reinterpret_cast<u32x4*>(xs + i) =
            glu8(*reinterpret_cast<const u32x4*>(xs + i), *reinterpret_cast<const u32x4*>(xs2 + i));
    } else if (pro == QD_PRO_RMSNORM) {
      float ss = 0.0f;
      for (int i = lane * 8; i < Kp; i += 512) ss = sumsq8(*reinterpret_cast<const u32x4*>(xs + i), ss);
      const float r = rms_inverse(wave_sum(ss), k, S.eps(g));
      for (int i = lane * 8; i < Kp; i += 512)
        *reinterpret_cast<u32x4*>(xs + i) =
            rms8(*reinterpret_cast<const u32x4*>(xs + i), r, *reinterpret_cast<const u32x4*>(xs2 + i));
    }
  } else {
    wait_stores();                                 // vmcnt(0): the data is in LDS
  }
  if (FMT == QD_FMT_INT4_G64) {
    // One 16-value run per lane, four runs' reads in flight before any sum:
    // this runs on the group boundary's critical path.
    const int runs = Kp / 16;
    const half2_t one2 = {(half_t)1.0f, (half_t)1.0f};
    for (int t0 = 0; t0 < runs; t0 += 256) {
      half8_t va[4], vb[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = min(t0 + 64 * u + lane, runs - 1);   // clamped read; result kept only if in range
        va[u] = *reinterpret_cast<const half8_t*>(xs + 16 * t);
        vb[u] = *reinterpret_cast<const half8_t*>(xs + 16 * t + 8);
      }
#pragma unroll
      for (int u = 0; u < 4; ++u) {
        const int t = t0 + 64 * u + lane;
        float sum = 0.0f;
#pragma unroll
        for (int e = 0; e < 8; e += 2) {
          sum = __builtin_amdgcn_fdot2((half2_t){va[u][e], va[u][e + 1]}, one2, sum, false);
          sum = __builtin_amdgcn_fdot2((half2_t){vb[u][e], vb[u][e + 1]}, one2, sum, false);
        }
        if (t < runs) {
          const int jj = t >> 4, within = t & 15;
          xsum[16 * jj + 4 * (within & 3) + (within >> 2)] = sum;
        }
      }
    }
  }
}

// Row-group rg of group g may belong to a different member in each lane, so
// the member lookup uses per-lane reads.
template <bool GLUE>
__device__ __forceinline__ void store_row(const Sched& S, int g, int rg, int row, float v) {
  int mi = S.mem0(g);
  const int last = mi + S.nmem(g) - 1;
  while (mi < last && rg >= S.rg_begin_l(mi + 1)) ++mi;
  const int64_t n = (int64_t)(rg - S.rg_begin_l(mi)) * kTileRows + row;
  if (n < S.n_l(mi))
    // Through a global pointer: a flat store would also count against the LDS
    // counter, making the next LDS wait wait for this store's acknowledgement.
    __hip_atomic_store((__attribute__((address_space(1))) uint16_t*)(S.y_l(mi) + n),
                       GLUE ? epilogue_bits(v, S.epi_l(mi)) : __builtin_bit_cast(uint16_t, (half_t)v),
                       __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Up to 16 token rows of row-group rg: lane (gq, rho) holds tokens 4 gq + i
// of weight row rho (the MFMA output layout).
template <int FMT>
__device__ __forceinline__ void store_rows16(const PlanArgs& p, const Sched& S, int g, int rg,
                                             int lane, float4_t v) {
  int mi = S.mem0(g);
  const int last = mi + S.nmem(g) - 1;
  while (mi < last && rg >= S.rg_begin(mi + 1)) ++mi;
  const int gq = lane >> 4, rho = lane & 15;
  const int64_t n = (int64_t)(rg - S.rg_begin(mi)) * kTileRows + rho;
  if (n >= S.n(mi)) return;
  uint16_t* const y = S.y(mi);
  uint16_t* const yt = S.yt(mi);
  const int64_t ld = S.ld(mi);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = 4 * gq + i;
    if (tok < p.m) {
      const uint16_t h = __builtin_bit_cast(uint16_t, (half_t)v[i]);
      __hip_atomic_store((__attribute__((address_space(1))) uint16_t*)(y + tok * ld + n), h,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The later group reading these outputs as its x finds them here in
      // matrix-core order too.
      if (yt)
        __hip_atomic_store((__attribute__((address_space(1))) uint16_t*)(yt + xt_index<FMT>(n, tok)),
                           h, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// Spin (bounded) until the compute waves have counted `want` tiles against
// row-group slot `seg`.  After one timed-out wait (an error) later waits are
// skipped.
__device__ __forceinline__ void wait_count(const PlanArgs& p, const uint32_t* cnt, int seg,
                                           uint32_t want, bool& dead) {
  for (uint32_t spins = 0; !dead && lds_get(cnt + seg) < want; ++spins) {
    if (spins > p.spin_limit) {
      atomicOr(p.err, 2u);
      dead = true;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
}

// Reduce the compute waves' partials of group g row-group by row-group, as
// each row-group's last tile is counted, and write its rows.  The sum over a
// row-group's tiles is taken in a fixed order whichever wave computed which
// tile (one row: tiles t = q mod 4 per quarter-wave, then the four quarters;
// up to 16 rows: each lane its float4 over the tiles in order), so results
// are deterministic.
template <int FMT, bool GLUE, int MT>
__device__ void finish_group(const PlanArgs& p, const Sched& S, int g, int lane, const float* red,
                             uint32_t* cnt, int* stalled, bool& dead) {
  const int ntiles = S.tiles(g);
  if (ntiles == 0) {
    if (lane == 0) lds_put(stalled, g);
    return;
  }
  const int J = S.J(g);
  const int rg0 = S.rg0(g), nseg = S.nseg(g);
  const int row = lane & 15, q = lane >> 4;
  for (int s = 0; s < nseg; ++s) {
    wait_count(p, cnt, s, (uint32_t)J, dead);
    if (s == nseg - 1 && lane == 0) lds_put(stalled, g);   // every tile of g is in
    if constexpr (MT != 1) {
      // Each lane sums its float4 over the row-group's tiles in tile order.
      const float4_t* r4 = reinterpret_cast<const float4_t*>(red);
      float4_t sum = {0.0f, 0.0f, 0.0f, 0.0f};
      int r = s * J;
      const int rend = (s + 1) * J;
      // Four partials' reads ahead of their adds (same order of addition).
      for (; r + 4 <= rend; r += 4) {
        float4_t v[4];
#pragma unroll
        for (int u = 0; u < 4; ++u) v[u] = r4[(r + u) * 64 + lane];
#pragma unroll
        for (int u = 0; u < 4; ++u)
#pragma unroll
          for (int i = 0; i < 4; ++i) sum[i] += v[u][i];
      }
      for (; r < rend; ++r) {
        const float4_t v = r4[r * 64 + lane];
#pragma unroll
        for (int i = 0; i < 4; ++i) sum[i] += v[i];
      }
      if (lane == 0) cnt[s] = 0u;
      store_rows16<FMT>(p, S, g, rg0 + s, lane, sum);
      continue;
    }
    // This runs on the group's critical path for its last row-group: four
    // partials' reads ahead of their adds (same order of addition).
    float part = 0.0f;
    int r = s * J + q;
    const int rend = (s + 1) * J;
    for (; r + 12 < rend; r += 16) {
      float v[4];
#pragma unroll
      for (int u = 0; u < 4; ++u) v[u] = red[(r + 4 * u) * 16 + row];
#pragma unroll
      for (int u = 0; u < 4; ++u) part += v[u];
    }
    for (; r < rend; r += 4) part += red[r * 16 + row];
    const float sum = quad_reduce(part);
    if (lane == 0) cnt[s] = 0u;                // ready for the next group
    if (lane < 16) store_row<GLUE>(S, g, rg0 + s, row, sum);
  }
}

// Publish that this workgroup has finished every row it owes group g.
// When no later group of the step reads or rewrites the outputs, they need
// only be visible when the kernel ends, and the stamp goes out without
// waiting for the stores to complete.
__device__ __forceinline__ void publish(const PlanArgs& p, const Sched& S, int g, int w, int lane) {
  if (S.order(g) & kAckOutputs) wait_stores();              // outputs before the stamp
  if (lane == 0)
    __hip_atomic_store(&p.flags[w], stamp(p, g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every workgroup has published group g.  One poll is a single
// coherent read of all stamps (4 loads per lane cover up to 512 workgroups);
// kPollDepth polls are kept in flight.
constexpr int kMaxWorkgroups = 512;
// One poll in flight measured best (8B 1371 vs 1389 us with two, 1395 with
// three, 1419 with six): every poll is a device-coherent read that queues
// with the CU's weight loads and the other workgroups' polls.
#ifndef QD_POLL_DEPTH
#define QD_POLL_DEPTH 1
#endif
constexpr int kPollDepth = QD_POLL_DEPTH;

__device__ __forceinline__ void poll_stamps(__amdgpu_buffer_rsrc_t rf, int lane, u32x4 (&v)[4]) {
  // The clobbers keep the compiler from merging two polls of the same
  // addresses into one load or hoisting a poll out of the loop.
  asm volatile("" ::: "memory");
#pragma unroll
  for (int b = 0; b < 4; ++b) v[b] = bload16_coherent(rf, (uint32_t)(128 * b + 2 * lane) * 8);
  asm volatile("" ::: "memory");
}

__device__ __forceinline__ bool stamps_reached(const u32x4 (&v)[4], int G, int lane,
                                               unsigned long long target) {
  bool ok = true;
#pragma unroll
  for (int b = 0; b < 4; ++b) {
    const int i = 128 * b + 2 * lane;
    const unsigned long long s0 = ((unsigned long long)v[b][1] << 32) | v[b][0];
    const unsigned long long s1 = ((unsigned long long)v[b][3] << 32) | v[b][2];
    ok = ok && (i >= G || s0 >= target) && (i + 1 >= G || s1 >= target);
  }
  return __ballot(!ok) == 0ull;
}

// Sleeps of 512 cycles before the first poll (see wait_group), per path,
// measured: one token row, before a dependent group (8B chained step 1505
// with 2, 1543 with none; 1 and 4 took 1513 and 1516 us), and up to 16 token
// rows (8B step 2025 with 6, 2118 with none; 2, 4 and 8 took 2063, 2037 and
// 2023, the chained step 2065 with 6 and 2085 with 8).
#ifndef QD_POLL_DELAY
#define QD_POLL_DELAY 2
#endif
#ifndef QD_POLL_DELAY16
#define QD_POLL_DELAY16 6
#endif
__device__ void wait_group(const PlanArgs& p, int g, int lane, int delay) {
  if (__hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return;
  const unsigned long long target = stamp(p, g);
  // Past the G stamps the buffer reads zeros, which the check ignores.
  const __amdgpu_buffer_rsrc_t rf = make_rsrc(p.flags, (uint32_t)p.G * 8);
  // kPollDepth polls in flight: each check consumes the oldest and issues a
  // new one, so a stamp is seen about one poll interval after it lands.
  u32x4 v[kPollDepth][4];
  // Called straight after the workgroup's own stamp, a first poll would find
  // most stamps missing, and every poll is a device-coherent read queued with
  // the weight stream: wait a fraction of a microsecond first.  (When the
  // next activations are staged before the wait, that round trip already
  // spaces the poll out: no delay.)
  for (int d = 0; d < delay; ++d) __builtin_amdgcn_s_sleep(8);
#pragma unroll
  for (int i = 0; i < kPollDepth - 1; ++i) poll_stamps(rf, lane, v[i]);
  bool done = false;
  for (uint32_t spins = 0; !done; spins += kPollDepth) {
#pragma unroll
    for (int i = 0; i < kPollDepth; ++i) {
      poll_stamps(rf, lane, v[(i + kPollDepth - 1) % kPollDepth]);
      if (!done && stamps_reached(v[i], p.G, lane, target)) done = true;
    }
    if (!done && spins > p.spin_limit) {
      if (lane == 0) atomicOr(p.err, 1u);
      break;
    }
  }
  wait_stores();                  // no poll left in flight
  asm volatile("" ::: "memory");
}

template <int FMT, bool GLUE, int MT>
__device__ void control_wave(const PlanArgs& p, const Sched& S, int w, int lane, half_t* xs,
                             float* xsum, const float* red, uint32_t* cnt, int* stalled,
                             int* staged) {
  // The control wave is on every group's critical path: let it issue ahead of
  // the compute waves that share its SIMD.
  __builtin_amdgcn_s_setprio(3);
  // Group 0's activations: nothing of this launch has written anything yet
  // (earlier launches' writes are visible at kernel start).
  if constexpr (MT == 1) stage_group_x<FMT, GLUE, kPolicyDefault>(S, 0, lane, xs, xsum);
  wg_barrier();                   // activations of group 0 staged
  bool dead = false;
  for (int g = 0; g < p.ngroups; ++g) {
    finish_group<FMT, GLUE, MT>(p, S, g, lane, red, cnt, stalled, dead);
    publish(p, S, g, w, lane);
    if (g + 1 < p.ngroups) {
      // Activations no earlier group writes are staged while the stamps are
      // awaited; the others only once every workgroup has finished g.  The
      // compute waves start g + 1 after the barrier either way.
      // (MT > 1: the compute waves read the activations themselves.)
      const bool early = (S.order(g + 1) & kStageEarly) != 0;
      if (MT == 1 && early) stage_group_x<FMT, GLUE, kPolicyDefault>(S, g + 1, lane, xs, xsum);
      // A further row range of the same op(s) reads nothing group g writes,
      // and needs what g needed, which g's own boundary already waited for.
      if (!(S.order(g + 1) & kNoWait))
        wait_group(p, g, lane, MT > 1 ? QD_POLL_DELAY16 : early ? 0 : QD_POLL_DELAY);
      if (MT == 1 && !early) {
        if (S.order(g + 1) & kCleanLines) stage_group_x<FMT, GLUE, kPolicyDefault>(S, g + 1, lane, xs, xsum);
        else stage_group_x<FMT, GLUE>(S, g + 1, lane, xs, xsum);
      }
      if (lane == 0) lds_put(staged, g + 1);
      wg_barrier();               // activations of g + 1 staged
    }
  }
}

template <int FMT, int D, int R, int RS, bool GLUE, int MT, int U>
__global__ __launch_bounds__(kWaves * 64) void stack_kernel(PlanArgs p) {
  static_assert(R >= 0 && R < kCtl && RS >= 1, "at least one streaming wave");
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + p.x_bytes);
  float* red = reinterpret_cast<float*>(smem + p.x_bytes + p.xsum_bytes);
  uint32_t* cnt = reinterpret_cast<uint32_t*>(smem + p.x_bytes + p.xsum_bytes + p.red_bytes);
  uint8_t* tab = smem + p.x_bytes + p.xsum_bytes + p.red_bytes + p.cnt_bytes;
  uint32_t* next = reinterpret_cast<uint32_t*>(tab + p.tab_bytes);   // tile hand-out counter
  int* stalled = reinterpret_cast<int*>(next + 1);   // last group whose tiles are all computed
  int* staged = reinterpret_cast<int*>(next + 2);    // last group whose activations are staged
  const int w = blockIdx.x;
  const int wave = uni(threadIdx.x >> 6);
  const int lane = threadIdx.x & 63;

  // Copy this workgroup's schedule to LDS: group and member tables, and its
  // own column of the per-workgroup schedule.
  Sched S;
  S.g = reinterpret_cast<const PGroup*>(tab);
  S.m = reinterpret_cast<const PMember*>(tab + (size_t)p.ngroups * sizeof(PGroup));
  S.s = reinterpret_cast<const PSched*>(tab + (size_t)p.ngroups * sizeof(PGroup) +
                                        (size_t)p.nmem * sizeof(PMember));
  {
    u32x4* dst = reinterpret_cast<u32x4*>(tab);
    const u32x4* gsrc = reinterpret_cast<const u32x4*>(p.groups);
    const u32x4* msrc = reinterpret_cast<const u32x4*>(p.members);
    const int ng16 = p.ngroups * (int)(sizeof(PGroup) / 16);    // 16-byte units
    const int nm16 = p.nmem * (int)(sizeof(PMember) / 16);
    for (int i = threadIdx.x; i < ng16 + nm16 + p.ngroups; i += kWaves * 64) {
      u32x4 val;
      if (i < ng16) val = gsrc[i];
      else if (i < ng16 + nm16) val = msrc[i - ng16];
      else val = *reinterpret_cast<const u32x4*>(p.sched + (size_t)(i - ng16 - nm16) * p.G + w);
      dst[i] = val;
    }
    if (threadIdx.x == 0) {
      *next = 0u;
      *stalled = -1;
      *staged = 0;
    }
    for (int i = threadIdx.x; i < p.cnt_bytes / 4; i += kWaves * 64) cnt[i] = 0u;
  }
  __syncthreads();

  if (wave == kCtl) {
    control_wave<FMT, GLUE, MT>(p, S, w, lane, xs, xsum, red, cnt, stalled, staged);
  } else {
    const int last = p.ngroups - 1;
    const int total = S.off(last) + S.tiles(last);
    if (wave < kCtl - R)
      compute_wave<FMT, D, false, R, MT, U>(p, S, total, next, lane, xs, xsum, red, cnt, stalled, staged);
    else
      compute_wave<FMT, RS, true, R, MT, U>(p, S, total, next, lane, xs, xsum, red, cnt, stalled, staged);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Before a step with up to 16 token rows: copy the activations no group of
// the step writes into matrix-core order (see load_xblock), 256 chunks of 16
// bytes per workgroup, chunk-contiguous stores.  Chunks of token rows past m
// or past K are left as they are (zero since the plan was made).
struct XtJob {
  const uint16_t* x;    // [m, k]
  uint16_t* t;          // the copy
  int64_t k;
  int64_t first_block;  // first workgroup of this job
};

template <int FMT>
__global__ __launch_bounds__(256) void xt_copy_kernel(const XtJob* jobs, int njobs, int m) {
  int lo = 0, hi = njobs - 1;
  while (lo < hi) {
    const int mid = (lo + hi + 1) >> 1;
    if (jobs[mid].first_block <= (int64_t)blockIdx.x) lo = mid;
    else hi = mid - 1;
  }
  const XtJob jb = jobs[lo];
  // chunk c = (8 j + q) 64 + lane, lane = 16 gq + t
  const int64_t c = ((int64_t)blockIdx.x - jb.first_block) * 256 + threadIdx.x;
  const int tok = (int)(c & 15), gq = (int)((c >> 4) & 3), q = (int)((c >> 6) & 7);
  const int64_t k = (c >> 9) * kSuperK + kpos<FMT>(q, gq);
  if (tok >= m || k >= jb.k) return;
  const u32x4 v = *reinterpret_cast<const u32x4*>(jb.x + tok * jb.k + k);
  *reinterpret_cast<u32x4*>(jb.t + c * 8) = v;
}

// Streaming ring depth per format (tiles per streaming wave), measured.
#ifndef QD_PLAN_RING8
#define QD_PLAN_RING8 3
#endif
#ifndef QD_PLAN_RING4
#define QD_PLAN_RING4 2
#endif
constexpr int kRing8 = QD_PLAN_RING8;
constexpr int kRing4 = QD_PLAN_RING4;

}  // namespace

}  // namespace qd

// ---------------------------------------------------------------------------
// Plan object

struct qd_stack_plan {
  int device = 0;
  bool persistent = false;
  int fmt = 0;
  bool multi = false;                    // m > 1
  bool glue = false;                     // one token row with a prologue or an epilogue
  std::vector<qd::StackGroup> tail;      // groups replayed after the persistent kernel
  std::vector<qd::StackGroup> replay;    // launch-per-group fallback (K = 0, mixed formats, glue, ...)
  void* tables = nullptr;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
  void* xt = nullptr;                    // m > 1: activation copies in matrix-core order
  void* xt_jobs = nullptr;               // copies made before each step
  int xt_njobs = 0;
  int64_t xt_blocks = 0;
  qd::PlanArgs args{};
  size_t lds = 0;
  unsigned long long epoch = 0;
};

namespace qd {

namespace {

struct HostGroup {
  const uint16_t* x;
  int64_t k;
  int J;
  std::vector<PMember> mem;
  std::vector<int64_t> src;    // the step group each member comes from (outputs of one never overlap)
  std::vector<int64_t> yt_off; // m > 1: byte offset of each member's matrix-core copy in the plan's copies, or -1
  int R;
  const uint16_t* gamma;
  int pro;
  float eps;
  int32_t order = 0;
  int64_t xt_off = -1;         // m > 1: byte offset of the group's x copy, or -1
};

bool ranges_overlap(const void* a, uint64_t an, const void* b, uint64_t bn) {
  if (!a || !b || !an || !bn) return false;
  const uintptr_t a0 = (uintptr_t)a, b0 = (uintptr_t)b;
  return a0 < b0 + bn && b0 < a0 + an;
}

// Bytes a member's outputs span: m rows of n, ld apart.
uint64_t y_span(const PMember& pm, int64_t m) { return ((uint64_t)(m - 1) * pm.ld + pm.n) * 2; }

// Whole cache lines (128 bytes) holding [p, p + n), as [a, b).
struct Lines {
  uintptr_t a = 0, b = 0;
  bool hits(const Lines& o) const { return a < o.b && o.a < b; }
};
Lines lines_of(const void* p, uint64_t n) {
  if (!p || !n) return {};
  const uintptr_t a = (uintptr_t)p;
  return {a & ~(uintptr_t)127, (a + n + 127) & ~(uintptr_t)127};
}

// Boundary ordering from the buffers: a group's x may be read early unless
// an earlier group's output overlaps it; a group's stores must complete
// before its stamp if a later group's x or output overlaps one of its
// outputs.  Outputs within one group of the step are disjoint, also once the
// group is split into row ranges (whose byte spans interleave when m > 1).
void order_groups(std::vector<HostGroup>& gs, int64_t m, int64_t tbytes) {
  const size_t n = gs.size();
  for (size_t i = 0; i < n; ++i) {
    const uint64_t xb = (uint64_t)m * gs[i].k * 2 * (gs[i].pro == QD_PRO_GLU ? 2 : 1);
    bool early = true;
    for (size_t j = 0; j < i; ++j) {
      for (size_t b = 0; b < gs[j].mem.size(); ++b) {
        const PMember& pj = gs[j].mem[b];
        const uint64_t yj = y_span(pj, m);
        bool reads = ranges_overlap(gs[i].x, xb, pj.y, yj) ||
                     (gs[i].pro == QD_PRO_RMSNORM && ranges_overlap(gs[i].gamma, (uint64_t)gs[i].k * 2, pj.y, yj));
        bool rewrites = false;
        for (size_t a = 0; a < gs[i].mem.size(); ++a)
          rewrites = rewrites || (gs[i].src[a] != gs[j].src[b] &&
                                  ranges_overlap(gs[i].mem[a].y, y_span(gs[i].mem[a], m), pj.y, yj));
        if (reads) early = false;
        if (reads || rewrites) gs[j].order |= kAckOutputs;
      }
    }
    if (early) gs[i].order |= kStageEarly;
  }
  // A group whose x an earlier group writes may still read it through the
  // caches when no cache can hold a stale copy of its lines.  The caches
  // start each launch clean; the lines are then fetched fresh unless, before
  // the last group writing them, some access brought them in: an earlier
  // write, an activation read by an earlier group (after its own barrier), or
  // a weight read or early activation read (these happen at any point of the
  // step).  So one group of the step (all its row ranges) may write the
  // lines; its stores are disjoint byte ranges.  Checked per 128-byte line.
  auto acts = [&](const HostGroup& g, Lines out[2]) {
    out[0] = lines_of(g.x, (uint64_t)m * g.k * 2 * (g.pro == QD_PRO_GLU ? 2 : 1));
    out[1] = g.pro == QD_PRO_RMSNORM ? lines_of(g.gamma, (uint64_t)g.k * 2) : Lines{};
  };
  for (size_t i = 0; i < n; ++i) {
    if (gs[i].order & kStageEarly) continue;
    Lines ai[2];
    acts(gs[i], ai);
    auto touches = [&](const Lines& l) { return l.hits(ai[0]) || l.hits(ai[1]); };
    size_t last_write = 0;
    int64_t writer = -1;            // the step group writing the lines
    bool clean = true;
    for (size_t j = 0; j < i; ++j) {
      for (size_t b = 0; b < gs[j].mem.size(); ++b) {
        if (!touches(lines_of(gs[j].mem[b].y, y_span(gs[j].mem[b], m)))) continue;
        if (writer >= 0 && writer != gs[j].src[b]) clean = false;
        writer = gs[j].src[b];
        last_write = j;
      }
    }
    for (size_t j = 0; clean && j < n; ++j) {
      for (const PMember& pj : gs[j].mem)
        if (touches(lines_of(pj.blob, (uint64_t)ceil_div(pj.n, kTileRows) * gs[j].J * tbytes)))
          clean = false;
      if (j == i) continue;
      if ((gs[j].order & kStageEarly) || j <= last_write) {
        Lines aj[2];
        acts(gs[j], aj);
        if (touches(aj[0]) || touches(aj[1])) clean = false;
      }
    }
    if (clean) gs[i].order |= kCleanLines;
  }
}

// Split groups into row ranges of at most `tiles` tiles per workgroup (G
// workgroups), so that one range's 16 x 16 tile partials fit in LDS.  Each
// range is a group of its own whose members are the slices of the original
// members it covers; ranges after the first carry kNoWait.  False if a
// single row-group has more tiles than that.
bool split_rows(std::vector<HostGroup>& gs, int64_t tiles, int G, int64_t tbytes) {
  std::vector<HostGroup> out;
  for (HostGroup& hg : gs) {
    const int64_t per_wg = tiles / hg.J;
    if (per_wg < 1) return false;
    const int64_t piece = per_wg * G;
    if (hg.R <= piece) {
      out.push_back(std::move(hg));
      continue;
    }
    for (int64_t a = 0; a < hg.R; a += piece) {
      const int64_t b = std::min<int64_t>(hg.R, a + piece);
      HostGroup pg{hg.x, hg.k, hg.J, {}, {}, {}, 0, hg.gamma, hg.pro, hg.eps};
      pg.order = hg.order;
      pg.xt_off = hg.xt_off;
      for (size_t q = 0; q < hg.mem.size(); ++q) {
        const PMember& mm = hg.mem[q];
        const int64_t r0 = mm.rg_begin, r1 = r0 + ceil_div(mm.n, kTileRows);
        const int64_t lo = std::max(a, r0), hi = std::min(b, r1);
        if (lo >= hi) continue;
        const int64_t skip = lo - r0;   // row-groups of the member before this range
        PMember slice = mm;
        slice.blob = mm.blob + skip * hg.J * tbytes;
        slice.y = mm.y + skip * kTileRows;
        slice.n = std::min<int64_t>(mm.n - skip * kTileRows, (hi - lo) * kTileRows);
        slice.rg_begin = pg.R;
        pg.mem.push_back(slice);
        pg.src.push_back(hg.src[q]);
        pg.yt_off.push_back(hg.yt_off[q] < 0 ? -1 : hg.yt_off[q] + skip * kTileRows * 16 * 2);
        pg.R += (int)(hi - lo);
      }
      if (a > 0) pg.order |= kNoWait;
      out.push_back(std::move(pg));
    }
  }
  gs = std::move(out);
  return true;
}

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

// Reserve waves (and tiles each) per format, as measured on MI355X.  int8:
// 7 reserve waves of 2 tiles, the 8 streaming waves then sitting two to a
// SIMD; this was best for the 2B-, 4B- and 8B-shaped steps alike (15 to 50
// tiles per workgroup per group).  More reserve tiles run several groups
// ahead and are then not free for the next stall; fewer leave memory idle
// for part of it.  INT4: no reserve waves, and rings of 2 tiles per
// streaming wave (8B INT4 step 993-996 us; rings of 1, 3, 4 and 6 took 1098,
// 1043-1050, 1089-1104 and 1111 us; 2 x 4, 4 x 2 and 7 x 2 reserve tiles with
// rings of 2 took 1051-1059, 1021-1025 and 1095-1109 us).
#ifndef QD_PLAN_RESERVE4
#define QD_PLAN_RESERVE4 0
#endif
#ifndef QD_PLAN_RESERVE4_S
#define QD_PLAN_RESERVE4_S 4
#endif
constexpr int kReserveInt4 = QD_PLAN_RESERVE4, kReserveInt4S = QD_PLAN_RESERVE4_S;

#ifndef QD_PLAN_RESERVE8_R
#define QD_PLAN_RESERVE8_R 7
#endif
#ifndef QD_PLAN_RESERVE8_S
#define QD_PLAN_RESERVE8_S 2
#endif
constexpr int kReserve8R = QD_PLAN_RESERVE8_R, kReserve8S = QD_PLAN_RESERVE8_S;

// Up to 16 token rows (int8): each ring slot also holds an activation block,
// so rings are shorter.
#ifndef QD_PLAN_RING16
#define QD_PLAN_RING16 1
#endif
#ifndef QD_PLAN_RESERVE16_R
#define QD_PLAN_RESERVE16_R 7
#endif
#ifndef QD_PLAN_UNIT16
#define QD_PLAN_UNIT16 2
#endif
#ifndef QD_PLAN_RESERVE16_S
#define QD_PLAN_RESERVE16_S 1
#endif
// INT4 at up to 16 token rows: its own shape (tiles of 2304 rather than 4352
// bytes), measured on the 8B INT4 step (us): reserve waves of one unit
// 0 / 2 / 3 / 4 / 5 / 6 / 7 / 10 gave 1671 / 1608 / 1607 / 1621-1634 / 1630 /
// 1650 / 1709 / 2038 (from two boxes); units of 3 row-groups 1636 with 4
// reserve waves.  A ring of 2 units, two units per reserve wave and units of
// 4 spill registers.
#ifndef QD_PLAN_RING16_INT4
#define QD_PLAN_RING16_INT4 QD_PLAN_RING16
#endif
#ifndef QD_PLAN_RESERVE16_INT4_R
#define QD_PLAN_RESERVE16_INT4_R 3
#endif
#ifndef QD_PLAN_RESERVE16_INT4_S
#define QD_PLAN_RESERVE16_INT4_S QD_PLAN_RESERVE16_S
#endif
#ifndef QD_PLAN_UNIT16_INT4
#define QD_PLAN_UNIT16_INT4 QD_PLAN_UNIT16
#endif
// Row-groups per unit at up to 16 token rows.
constexpr int unit16(int fmt) { return fmt == QD_FMT_INT8_B32 ? QD_PLAN_UNIT16 : QD_PLAN_UNIT16_INT4; }
// Tiles per workgroup per group at up to 16 token rows: their 1 KB partials
// are held in LDS until the row-group is reduced.
#ifndef QD_PLAN_TILES16
#define QD_PLAN_TILES16 96
#endif

// One token row with glue: the staging applies the prologue in LDS and the
// row stores apply the epilogue (a separate instance, so steps without glue
// run the plain kernel).
const void* kernel_ptr(int fmt, bool multi, bool glue) {
  if (multi)
    return fmt == QD_FMT_INT8_B32
               ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, QD_PLAN_RING16, QD_PLAN_RESERVE16_R,
                                                             QD_PLAN_RESERVE16_S, false, 16, QD_PLAN_UNIT16>)
               : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT4_G64, QD_PLAN_RING16_INT4,
                                                             QD_PLAN_RESERVE16_INT4_R, QD_PLAN_RESERVE16_INT4_S,
                                                             false, 16, QD_PLAN_UNIT16_INT4>);
  if (fmt == QD_FMT_INT8_B32)
    return glue ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, kRing8, kReserve8R, kReserve8S, true, 1, 1>)
                : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, kRing8, kReserve8R, kReserve8S, false, 1, 1>);
  return glue ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT4_G64, kRing4, kReserveInt4, kReserveInt4S, true, 1, 1>)
              : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT4_G64, kRing4, kReserveInt4, kReserveInt4S, false, 1, 1>);
}

// The persistent step's tables, built on the host alone: the groups in step
// order with their boundary ordering, their row-range split at several token
// rows, the activation-copy slots, the per-workgroup schedules and the LDS
// the kernel needs, for G workgroups.  Copy addresses are byte offsets into
// the plan's copies until those exist.
struct PlanLayout {
  bool persistent = false;     // false: the whole step replays per-group launches
  int fmt = 0;
  bool multi = false, glue = false;
  int64_t split = 0;           // ops [0, split) run in the persistent kernel; the rest replay after it
  int G = 0;
  std::vector<PGroup> pg;
  std::vector<PMember> pm;
  std::vector<PSched> ps;      // [group][workgroup]
  std::vector<int64_t> xt_fix, yt_fix;   // per group / member: offset of its copy, or -1
  std::vector<XtJob> jobs;     // copies made before each step (t holds the offset)
  int64_t xt_total = 0, xt_blocks = 0;
  size_t x_bytes = 0, xsum_bytes = 0, red_bytes = 0, cnt_bytes = 0, tab_bytes = 0, lds = 0;
};

void layout_plan(const qd_linear_op* ops, int64_t n_ops, int64_t m, int G, PlanLayout* L) {
  *L = PlanLayout{};
  L->G = G;
  // Persistent walker: one format, no empty-K groups; one token row (with or
  // without glue), or up to 16 without glue.  The leading
  // groups that qualify run in the persistent kernel; from the first group
  // that does not (another format, say an fp16 head), the rest of the step
  // is replayed as per-group launches after it on the same stream.
  std::vector<HostGroup> groups;
  const bool multi = m > 1;
  bool glue = false;
  if (m < 1 || m > 16 || G < 1 || G > kMaxWorkgroups) return;
  int fmt = 0;
  int64_t split = n_ops;
  for (int64_t i = 0; i < n_ops;) {
    int64_t e = i + 1;
    while (e < n_ops && ops[e].group == ops[i].group) ++e;
    HostGroup hg{ops[i].x, ops[i].w.k, (int)ceil_div(ops[i].w.k, kSuperK), {}, {}, {}, 0,
                 ops[i].gamma, ops[i].prologue, ops[i].eps};
    bool gok = true, gglue = false;
    int gfmt = fmt;
    for (int64_t q = i; q < e; ++q) {
      if (ops[q].w.n == 0) continue;
      if (ops[q].w.k == 0) gok = false;
      if (gfmt == 0) gfmt = ops[q].w.fmt;
      if (ops[q].w.fmt != gfmt) gok = false;
      if (gfmt != QD_FMT_INT8_B32 && gfmt != QD_FMT_INT4_G64) gok = false;   // fp16: replay
      // Glue (a prologue or an epilogue): at one token row only.
      if (ops[q].prologue != QD_PRO_NONE || ops[q].epilogue != QD_EPI_NONE) {
        gglue = true;
        if (multi) gok = false;
      }
      hg.mem.push_back(PMember{static_cast<const uint8_t*>(ops[q].w.data), ops[q].y, ops[q].w.n,
                               hg.R, ops[q].epilogue, ops[q].w.n, nullptr});
      hg.src.push_back(i);
      hg.yt_off.push_back(-1);
      hg.R += (int)ceil_div(ops[q].w.n, kTileRows);
    }
    if (!gok) {
      split = i;
      break;
    }
    fmt = gfmt;
    glue = glue || gglue;
    if (!hg.mem.empty()) groups.push_back(std::move(hg));
    i = e;
  }
  if (groups.empty()) return;
  order_groups(groups, m, tile_bytes(fmt));

  // Several token rows: copies of the activations in matrix-core order.  An
  // activation no group writes is copied before the step; one that is
  // exactly an earlier op's whole output (the last write to any of its
  // bytes) is written in that order by the op itself.  Other activations are
  // read in place.
  std::vector<XtJob> jobs;
  int64_t xt_total = 0;
  if (multi) {
    std::map<std::pair<const void*, int64_t>, int64_t> early_slots;
    std::map<std::pair<size_t, size_t>, int64_t> out_slots;
    auto new_slot = [&](int J) {
      const int64_t off = xt_total;
      xt_total += (int64_t)align_up((size_t)J * 8192, 256);
      return off;
    };
    for (size_t g = 0; g < groups.size(); ++g) {
      HostGroup& hg = groups[g];
      if (hg.order & kStageEarly) {
        const auto key = std::make_pair((const void*)hg.x, hg.k);
        auto it = early_slots.find(key);
        if (it == early_slots.end()) {
          it = early_slots.emplace(key, new_slot(hg.J)).first;
          jobs.push_back(XtJob{hg.x, reinterpret_cast<uint16_t*>((uintptr_t)it->second), hg.k, 0});
        }
        hg.xt_off = it->second;
        continue;
      }
      size_t p = SIZE_MAX, q = 0;
      for (size_t j = 0; j < g; ++j)
        for (size_t b = 0; b < groups[j].mem.size(); ++b)
          if (ranges_overlap(hg.x, (uint64_t)m * hg.k * 2, groups[j].mem[b].y, y_span(groups[j].mem[b], m))) {
            p = j;
            q = b;
          }
      if (p == SIZE_MAX) continue;
      const PMember& pq = groups[p].mem[q];
      if ((const void*)pq.y != (const void*)hg.x || pq.n != hg.k || pq.ld != hg.k) continue;
      // The copy's order repeats every 256 rows, and a row range cut out of
      // the member (split_rows, below) addresses its part of the copy by a
      // plain offset: so every cut must fall a whole number of 256-row
      // blocks into the member, else the member writes no copy.
      const int64_t piece = (int64_t)(QD_PLAN_TILES16 / groups[p].J) * G;
      const int64_t r0 = pq.rg_begin, r1 = r0 + ceil_div(pq.n, kTileRows);
      bool cuts_aligned = true;
      for (int64_t a = piece; piece > 0 && a < groups[p].R; a += piece)
        if (a > r0 && a < r1 && (a - r0) % (256 / kTileRows) != 0) cuts_aligned = false;
      if (!cuts_aligned) continue;
      auto it = out_slots.find(std::make_pair(p, q));
      if (it == out_slots.end()) it = out_slots.emplace(std::make_pair(p, q), new_slot(hg.J)).first;
      groups[p].yt_off[q] = it->second;
      hg.xt_off = it->second;
    }
  }
  if (multi && !split_rows(groups, QD_PLAN_TILES16, G, tile_bytes(fmt))) return;
  const int ng = (int)groups.size();
  L->pg.resize(ng);
  L->ps.resize((size_t)ng * G);
  std::vector<int32_t> off(G, 0);
  int maxJ = 1, maxXH = 512, maxRel = 1, maxSeg = 1;
  for (int g = 0; g < ng; ++g) {
    HostGroup& hg = groups[g];
    const int64_t J = hg.J, R = hg.R, T = R * J;
    // A step the persistent walker cannot hold (tile counts past int32)
    // replays per-group launches instead.
    if (T > (int64_t)INT32_MAX / 2) return;
    L->pg[g] = PGroup{hg.x, hg.gamma, nullptr, hg.k, hg.J, hg.R, (int32_t)L->pm.size(), (int32_t)hg.mem.size(),
                      hg.pro, hg.eps, hg.order, 0};
    L->xt_fix.push_back(hg.xt_off);
    for (size_t b = 0; b < hg.mem.size(); ++b) {
      L->pm.push_back(hg.mem[b]);
      L->yt_fix.push_back(hg.yt_off[b]);
    }
    maxJ = std::max(maxJ, hg.J);
    // halves of LDS the staging writes: x's span, and the second operand's
    maxXH = std::max(maxXH, (hg.pro == QD_PRO_NONE ? 1 : 2) * x_span(hg.J * kSuperK));
    // Tile ranges per workgroup: whole row-groups, spread evenly; when the
    // group has fewer row-groups than workgroups some get none (their waves
    // go on prefetching the next groups).  Splitting a row-group across
    // workgroups would put a cross-workgroup combine, one more device-wide
    // round trip, on the group's critical path; measured, that costs more
    // than the uneven split.
    for (int w = 0; w < G; ++w) {
      // Contiguous row-groups: each workgroup streams one contiguous range.
      // (Interleaving them, row-group w + i G to workgroup w, measured 2-11%
      // slower: the contiguous streams keep DRAM pages open.)
      // Several token rows: the sequence holds units of unit16(fmt) row-groups.
      const int64_t r0 = (int64_t)w * R / G, nrg = (int64_t)(w + 1) * R / G - r0;
      const int64_t n = (multi ? ceil_div(nrg, (int64_t)unit16(fmt)) : nrg) * J;
      L->ps[(size_t)g * G + w] = PSched{(int32_t)n, off[w], (int32_t)r0, (int32_t)nrg};
      if (nrg == 0) continue;
      off[w] += (int32_t)n;
      maxRel = std::max<int>(maxRel, (int)(nrg * J));
      maxSeg = std::max<int>(maxSeg, (int)nrg);
    }
  }
  // Several token rows: no staged activations, and 16 x 16 partials per tile.
  L->x_bytes = multi ? 0 : (size_t)maxXH * 2;      // a multiple of 1024
  L->xsum_bytes = fmt == QD_FMT_INT4_G64 && !multi ? align_up((size_t)maxJ * 16 * 4, 16) : 0;
  L->red_bytes = align_up((size_t)maxRel * 16 * 4 * (multi ? 16 : 1), 16);
  L->cnt_bytes = align_up((size_t)maxSeg * 4, 16);
  L->tab_bytes = (size_t)ng * sizeof(PGroup) + L->pm.size() * sizeof(PMember) + (size_t)ng * sizeof(PSched);
  L->lds = L->x_bytes + L->xsum_bytes + L->red_bytes + L->cnt_bytes + L->tab_bytes + 16;   // + counter, stall flag
  int64_t blocks = 0;
  for (XtJob& jb : jobs) {
    jb.first_block = blocks;
    blocks += 2 * ceil_div(jb.k, kSuperK);         // 512 chunks per super-block
  }
  L->jobs = std::move(jobs);
  L->xt_total = xt_total;
  L->xt_blocks = blocks;
  L->fmt = fmt;
  L->multi = multi;
  L->glue = glue;
  L->split = split;
  L->persistent = true;
}

}  // namespace

qd_status plan_create(const qd_linear_op* ops, int64_t n_ops, int64_t m, qd_stack_plan** out) {
  std::vector<StackGroup> replay;
  qd_status st = build_groups(ops, n_ops, m, &replay);
  if (st != QD_OK) return st;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QD_EDEVICE;
  qd_stack_plan* plan = new (std::nothrow) qd_stack_plan;
  if (!plan) return QD_ELAUNCH;
  plan->device = dev;
  // Whatever the persistent kernel cannot take replays per-group launches.
  auto fallback = [&]() {
    plan->replay = std::move(replay);
    *out = plan;
    return QD_OK;
  };
  int cus = 0;
  if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess) {
    (void)hipGetLastError();
    return fallback();
  }
  PlanLayout L;
  layout_plan(ops, n_ops, m, cus, &L);
  if (!L.persistent) return fallback();
  std::vector<StackGroup> tail;
  if (L.split < n_ops && build_groups(ops + L.split, n_ops - L.split, m, &tail) != QD_OK) return fallback();
  const int G = L.G, ng = (int)L.pg.size();
  std::vector<PGroup>& pg = L.pg;
  std::vector<PMember>& pm = L.pm;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    delete plan;
    return QD_EDEVICE;
  }
  // LDS beyond one CU's: replay.
  const void* kfn = kernel_ptr(L.fmt, L.multi, L.glue);
  const size_t lds = L.lds;
  const size_t lds_max = std::max<size_t>(prop.sharedMemPerBlock, prop.maxSharedMemoryPerMultiProcessor);
  if (lds > lds_max) return fallback();
  if (lds > 65536 &&
      hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    (void)hipGetLastError();
    return fallback();
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, kWaves * 64, lds) != hipSuccess ||
      per_cu < 1) {
    (void)hipGetLastError();
    return fallback();
  }

  // The activation copies (zeroed once: token rows past m and K positions
  // past K stay zero) and the table of copies made before each step.
  if (L.xt_total > 0) {
    void* dj = nullptr;
    if (hipMalloc(&plan->xt, (size_t)L.xt_total) != hipSuccess ||
        hipMemset(plan->xt, 0, (size_t)L.xt_total) != hipSuccess ||
        (!L.jobs.empty() && hipMalloc(&dj, sizeof(XtJob) * L.jobs.size()) != hipSuccess)) {
      if (plan->xt) (void)hipFree(plan->xt);
      delete plan;
      return QD_ELAUNCH;
    }
    uint8_t* const xb = static_cast<uint8_t*>(plan->xt);
    for (XtJob& jb : L.jobs) jb.t = reinterpret_cast<uint16_t*>(xb + reinterpret_cast<uintptr_t>(jb.t));
    if (!L.jobs.empty() &&
        hipMemcpy(dj, L.jobs.data(), sizeof(XtJob) * L.jobs.size(), hipMemcpyHostToDevice) != hipSuccess) {
      (void)hipFree(plan->xt);
      (void)hipFree(dj);
      delete plan;
      return QD_ELAUNCH;
    }
    plan->xt_jobs = dj;
    plan->xt_njobs = (int)L.jobs.size();
    plan->xt_blocks = L.xt_blocks;
    for (int g = 0; g < ng; ++g)
      if (L.xt_fix[g] >= 0) pg[g].xt = reinterpret_cast<const uint16_t*>(xb + L.xt_fix[g]);
    for (size_t i = 0; i < pm.size(); ++i)
      if (L.yt_fix[i] >= 0) pm[i].yt = reinterpret_cast<uint16_t*>(xb + L.yt_fix[i]);
  }

  // Device tables, then scratch.
  const size_t o_groups = 0;
  const size_t o_mem = align_up(o_groups + sizeof(PGroup) * ng, 256);
  const size_t o_sched = align_up(o_mem + sizeof(PMember) * pm.size(), 256);
  const size_t t_bytes = align_up(o_sched + sizeof(PSched) * L.ps.size(), 256);
  const size_t s_flags = 0;
  const size_t s_err = align_up(sizeof(unsigned long long) * G, 256);
  const size_t s_bytes = s_err + 256;
  std::vector<uint8_t> host(t_bytes, 0);
  memcpy(host.data() + o_groups, pg.data(), sizeof(PGroup) * ng);
  memcpy(host.data() + o_mem, pm.data(), sizeof(PMember) * pm.size());
  memcpy(host.data() + o_sched, L.ps.data(), sizeof(PSched) * L.ps.size());
  if (hipMalloc(&plan->tables, t_bytes) != hipSuccess ||
      hipMalloc(&plan->scratch, s_bytes) != hipSuccess ||
      hipMemcpy(plan->tables, host.data(), t_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(plan->scratch, 0, s_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    if (plan->tables) (void)hipFree(plan->tables);
    if (plan->scratch) (void)hipFree(plan->scratch);
    if (plan->xt) (void)hipFree(plan->xt);
    if (plan->xt_jobs) (void)hipFree(plan->xt_jobs);
    delete plan;
    return QD_ELAUNCH;
  }
  uint8_t* tb = static_cast<uint8_t*>(plan->tables);
  uint8_t* sb = static_cast<uint8_t*>(plan->scratch);
  PlanArgs& a = plan->args;
  a.groups = reinterpret_cast<const PGroup*>(tb + o_groups);
  a.members = reinterpret_cast<const PMember*>(tb + o_mem);
  a.sched = reinterpret_cast<const PSched*>(tb + o_sched);
  a.flags = reinterpret_cast<unsigned long long*>(sb + s_flags);
  a.err = reinterpret_cast<uint32_t*>(sb + s_err);
  a.ngroups = ng;
  a.nmem = (int32_t)pm.size();
  a.G = G;
  a.x_bytes = (int32_t)L.x_bytes;
  a.xsum_bytes = (int32_t)L.xsum_bytes;
  a.red_bytes = (int32_t)L.red_bytes;
  a.cnt_bytes = (int32_t)L.cnt_bytes;
  a.tab_bytes = (int32_t)L.tab_bytes;
  a.m = (int32_t)m;
  a.spin_limit = kSpinLimit;
  plan->scratch_bytes = s_bytes;
  plan->lds = lds;
  plan->fmt = L.fmt;
  plan->multi = L.multi;
  plan->glue = L.glue;
  plan->tail = std::move(tail);
  plan->persistent = true;
  *out = plan;
  return QD_OK;
}

qd_status plan_describe(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t workgroups,
                        int64_t* out, int64_t cap, int64_t* out_len) {
  if (workgroups < 1 || workgroups > kMaxWorkgroups) return QD_EINVAL;
  std::vector<StackGroup> replay;
  qd_status st = build_groups(ops, n_ops, m, &replay);
  if (st != QD_OK) return st;
  PlanLayout L;
  layout_plan(ops, n_ops, m, workgroups, &L);
  if (L.persistent) {
    std::vector<StackGroup> tail;
    if (L.split < n_ops && build_groups(ops + L.split, n_ops - L.split, m, &tail) != QD_OK) L = PlanLayout{};
  }
  std::vector<int64_t> v = {1, L.persistent, L.fmt, m, L.glue, L.persistent ? L.split : 0,
                            (int64_t)L.pg.size(), (int64_t)L.pm.size(), L.G, L.xt_total,
                            (int64_t)L.jobs.size(), (int64_t)L.lds, (int64_t)L.x_bytes,
                            (int64_t)L.red_bytes, (int64_t)L.cnt_bytes, (int64_t)L.tab_bytes};
  auto addr = [](const void* p) { return (int64_t)(uintptr_t)p; };
  for (size_t g = 0; g < L.pg.size(); ++g) {
    const PGroup& p = L.pg[g];
    v.insert(v.end(), {addr(p.x), addr(p.gamma), p.k, p.J, p.R, p.mem0, p.n_mem, p.pro, p.order, L.xt_fix[g]});
  }
  for (size_t i = 0; i < L.pm.size(); ++i) {
    const PMember& p = L.pm[i];
    v.insert(v.end(), {addr(p.blob), addr(p.y), p.n, p.rg_begin, p.epi, p.ld, L.yt_fix[i]});
  }
  for (const PSched& s : L.ps) v.insert(v.end(), {s.n, s.off, s.rg0, s.nseg});
  for (const XtJob& j : L.jobs)
    v.insert(v.end(), {addr(j.x), (int64_t)reinterpret_cast<uintptr_t>(j.t), j.k, j.first_block});
  *out_len = (int64_t)v.size();
  if (!out) return QD_OK;                           // a size query
  if (cap < (int64_t)v.size()) return QD_ESHAPE;
  std::copy(v.begin(), v.end(), out);
  return QD_OK;
}

qd_status plan_run(qd_stack_plan* plan, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return QD_EDEVICE;
  if (!plan->persistent) return launch_groups(plan->replay, s) == hipSuccess ? QD_OK : QD_ELAUNCH;
  if (plan->xt_njobs > 0) {
    if (plan->fmt == QD_FMT_INT8_B32)
      hipLaunchKernelGGL(xt_copy_kernel<QD_FMT_INT8_B32>, dim3((unsigned)plan->xt_blocks), dim3(256), 0, s,
                         static_cast<const XtJob*>(plan->xt_jobs), plan->xt_njobs, (int)plan->args.m);
    else
      hipLaunchKernelGGL(xt_copy_kernel<QD_FMT_INT4_G64>, dim3((unsigned)plan->xt_blocks), dim3(256), 0, s,
                         static_cast<const XtJob*>(plan->xt_jobs), plan->xt_njobs, (int)plan->args.m);
    if (hipGetLastError() != hipSuccess) return QD_ELAUNCH;
  }
  plan->args.epoch = ++plan->epoch;
  void* kargs[] = {&plan->args};
  const hipError_t e = hipLaunchCooperativeKernel(kernel_ptr(plan->fmt, plan->multi, plan->glue), dim3(plan->args.G),
                                                  dim3(kWaves * 64), kargs, (unsigned)plan->lds, s);
  if (e != hipSuccess) {
    --plan->epoch;
    return QD_ELAUNCH;
  }
  // The groups after the persistent part, in stream order behind it.
  if (!plan->tail.empty() && launch_groups(plan->tail, s) != hipSuccess) return QD_ELAUNCH;
  return QD_OK;
}

qd_status plan_error(qd_stack_plan* plan, int32_t* out_error) {
  *out_error = 0;
  if (!plan->persistent) return QD_OK;
  uint32_t e = 0;
  if (hipMemcpy(&e, plan->args.err, sizeof(e), hipMemcpyDeviceToHost) != hipSuccess)
    return QD_ELAUNCH;
  *out_error = (int32_t)e;
  if (e != 0) {
    // A timed-out wait leaves the counters inconsistent: start over.
    if (hipMemset(plan->scratch, 0, plan->scratch_bytes) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
      return QD_ELAUNCH;
    plan->epoch = 0;
  }
  return QD_OK;
}

bool plan_is_persistent(const qd_stack_plan* plan) { return plan->persistent; }

void plan_set_spin_limit(qd_stack_plan* plan, uint32_t polls) { plan->args.spin_limit = polls; }

void plan_destroy(qd_stack_plan* plan) {
  if (!plan) return;
  if (plan->tables) (void)hipFree(plan->tables);
  if (plan->scratch) (void)hipFree(plan->scratch);
  if (plan->xt) (void)hipFree(plan->xt);
  if (plan->xt_jobs) (void)hipFree(plan->xt_jobs);
  delete plan;
}

}  // namespace qd
