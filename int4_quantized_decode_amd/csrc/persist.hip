// Persistent decode-step kernel: one launch walks every group of the step.
//
// Decode streams every quantized weight once per token (Qwen3-VL 4B/8B Core
// AI cards, Measured paragraph), so a step's time is the weight stream plus
// whatever stalls it.  Per-group launches stall it at every group boundary:
// the next kernel starts loading only after the previous one drains.  Here the
// weight stream keeps going across group boundaries:
//
//   * one workgroup per CU (cooperative launch, all co-resident), 16 waves:
//     15 compute waves and 1 control wave.  The workgroup's share of every
//     group's schedule lives in LDS, so no wave waits on a memory round trip
//     to find its next tiles;
//   * a group's tiles (row-group major) are split into one range per
//     workgroup, on row-group boundaries whenever the group has at least one
//     row-group per workgroup; each compute wave takes a contiguous part of
//     the range;
//   * each compute wave keeps a ring of D tiles in registers, reloading a
//     slot as soon as it is consumed and following its tile sequence across
//     group boundaries, so weights of the next groups are in flight while the
//     current group completes;
//   * a group's activation vector is read only after every workgroup has
//     published that it finished the group before (one completion stamp per
//     workgroup, polled with a single 2 KiB read), so an op may consume an
//     earlier op's output;
//   * compute waves issue no global stores or atomics.  Per-wave row partial
//     sums go to LDS; the control wave reduces them, writes outputs, combines
//     row-groups split across workgroups (fixed-order sums: deterministic),
//     publishes completion and stages the next activation vector.
//
// Data another workgroup reads (outputs, split-row-group partials, stamps) is
// written with device-coherent stores and read with device-coherent loads,
// which are served at the level all of the device's L2s share; a writer waits
// for its data stores to complete before it publishes a stamp.  No L2-wide
// write-back or invalidate is issued.
//
// Waits are bounded: a wait that exceeds its spin limit sets an error word
// and every later wait is skipped, so the kernel always finishes.
#include <algorithm>
#include <cstring>
#include <new>
#include <vector>

#include "stack.h"
#include "tiles.h"

namespace qd {

namespace {

constexpr int kWaves = 16;
constexpr int kWc = 15;                 // compute waves
constexpr int kCtl = 15;                // the control wave
constexpr uint32_t kSpinLimit = 1u << 20;   // polls (each a device-coherent round trip): ~1 s

struct PGroup {         // 32 bytes
  const uint16_t* x;
  int64_t k;
  int32_t J;            // super-blocks per row
  int32_t R;            // row-groups in the group
  int32_t mem0;         // first member in the member table
  int32_t n_mem;
};

struct PMember {        // 32 bytes
  const uint8_t* blob;
  uint16_t* y;
  int64_t n;
  int32_t rg_begin;     // first row-group of this member within its group
  int32_t pad;
};

struct PSched {         // 32 bytes: one workgroup's part of one group
  int32_t a, b;         // tile range [a, b)
  int32_t wf0, nc0;     // first row-group: first contributing workgroup, contributors
  int32_t wf1, nc1;     // last row-group: same
  int32_t off;          // tiles of this workgroup in the groups before this one
  int32_t rg0;          // a / J: first row-group touched
};

static_assert(sizeof(PGroup) == 32 && sizeof(PMember) == 32 && sizeof(PSched) == 32,
              "schedule records are copied to LDS in 16-byte units");

struct PlanArgs {
  const PGroup* groups;       // [ngroups]
  const PMember* members;     // [nmem]
  const PSched* sched;        // [ngroups][G]
  unsigned long long* flags;  // [G] completion stamps
  unsigned long long* slots;  // [G][2][16] split-row-group partials: (stamp << 32) | float bits
  uint32_t* err;
  unsigned long long epoch;   // runs so far, including this one
  int32_t ngroups;
  int32_t nmem;
  int32_t G;
  int32_t x_bytes;            // LDS layout: x | xsum | red | groups | members | sched
  int32_t xsum_bytes;
  int32_t red_bytes;
  int32_t tab_bytes;
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
  __device__ int64_t k(int gi) const { return (int64_t)uni((int)g[gi].k); }
  __device__ int a(int gi) const { return uni(s[gi].a); }
  __device__ int b(int gi) const { return uni(s[gi].b); }
  __device__ int off(int gi) const { return uni(s[gi].off); }
  __device__ int rg0(int gi) const { return uni(s[gi].rg0); }
  __device__ int rg_begin(int mi) const { return uni(m[mi].rg_begin); }
  __device__ const uint8_t* blob(int mi) const { return uni_ptr(m[mi].blob); }
  __device__ uint16_t* y(int mi) const { return uni_ptr(m[mi].y); }
  __device__ int64_t n(int mi) const { return (int64_t)uni((int)m[mi].n); }
  // Per-lane reads, for a member index that may differ between lanes.
  __device__ int rg_begin_l(int mi) const { return m[mi].rg_begin; }
  __device__ uint16_t* y_l(int mi) const { return m[mi].y; }
  __device__ int64_t n_l(int mi) const { return m[mi].n; }
};

// Tile hand-out.  A workgroup's tiles of all groups form one sequence
// (group by group, row-group major); compute waves take the next index from
// an LDS counter whenever a ring slot frees.  Tiles are therefore fetched in
// sequence order whatever the waves' relative progress, so a group completes
// when its last tile lands, and loads for the next groups queue behind it.
struct TileRef {
  int g;      // group (ngroups: no tile)
  int j;      // super-block within the row
  int rel;    // tile index relative to the first row-group of the range (t - rg0 J)
};

struct IssueCursor {
  int g;                // current group (-1 before the first)
  int off_next;         // sequence index where the next group starts
  int t, rg, j;         // last issued tile of the group, as (row-group, super-block)
  int J, rg0, a;
  int mem, mem_last;
};

template <int FMT>
__device__ __forceinline__ typename Fmt<FMT>::Tile issue(const Sched& S, int ngroups, int total,
                                                         uint32_t* next, IssueCursor& c,
                                                         TileRef& ref, int lane) {
  constexpr int T = Fmt<FMT>::kT;
  uint32_t got = 0;
  if (lane == 0) got = atomicAdd(next, 1u);
  const int idx = uni((int)got);
  const uint8_t* base = nullptr;
  uint32_t nbytes = 0;
  ref.g = ngroups;
  if (idx < total) {
    while (idx >= c.off_next) {                       // enter the group holding idx
      ++c.g;
      c.J = S.J(c.g);
      c.a = S.a(c.g);
      c.rg0 = S.rg0(c.g);
      c.off_next = c.g + 1 < ngroups ? S.off(c.g + 1) : total;
      c.t = c.a;
      c.rg = c.rg0;
      c.j = c.a - c.rg0 * c.J;
      c.mem = S.mem0(c.g);
      c.mem_last = c.mem + S.nmem(c.g) - 1;
    }
    const int t = c.a + idx - S.off(c.g);
    c.j += t - c.t;
    c.t = t;
    while (c.j >= c.J) {
      c.j -= c.J;
      ++c.rg;
    }
    while (c.mem < c.mem_last && c.rg >= S.rg_begin(c.mem + 1)) ++c.mem;
    base = S.blob(c.mem) + (int64_t)(t - S.rg_begin(c.mem) * c.J) * T;
    nbytes = T;
    ref.g = c.g;
    ref.j = c.j;
    ref.rel = t - c.rg0 * c.J;
  }
  return Fmt<FMT>::load(make_rsrc(base, nbytes), lane);
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

// Keep a load where it is written: the scheduler may not move code across
// the barrier, and the memory clobber stops earlier passes from sinking the
// load towards its first use (which would empty the ring).
#define QD_PIN_ISSUE()                  \
  do {                                  \
    __builtin_amdgcn_sched_barrier(0);  \
    asm volatile("" ::: "memory");      \
  } while (0)

template <int FMT, int D>
__device__ void compute_wave(const PlanArgs& p, const Sched& S, int total, uint32_t* next,
                             int lane, const half_t* xs, const float* xsum, float* red) {
  (void)p;
  using Tile = typename Fmt<FMT>::Tile;
  const int ng = p.ngroups;
  const int g4 = lane >> 4;
  IssueCursor ic{-1, 0, 0, 0, 0, 1, 0, 0, 0, 0};
  Tile ring[D];
  TileRef ref[D];
#pragma unroll
  for (int s = 0; s < D; ++s) {
    ring[s] = issue<FMT>(S, ng, total, next, ic, ref[s], lane);
    QD_PIN_ISSUE();
  }
  // Barriers: "activations staged" on entering a group, "group done" on
  // leaving it; every wave passes both for every group, in order.
  int cg = -1;
  auto settle_to = [&](int g) {
    while (cg < g) {
      if (cg >= 0) wg_barrier();
      ++cg;
      if (cg < ng) wg_barrier();
    }
  };
  // Each tile's row partials go to their own LDS slot: the sum over tiles is
  // then taken in a fixed order, whichever wave computed which tile.
  // The ring is consumed and refilled in slot order with a single loop exit,
  // so each compute waits only for its own slot's loads.
  for (;;) {
#pragma unroll
    for (int s = 0; s < D; ++s) {
      if (ref[s].g < ng) {
        settle_to(ref[s].g);
        const float part = quad_reduce(tile_dot<FMT>(ring[s], xs, xsum, ref[s].j, g4, 0.0f));
        if (lane < 16) red[ref[s].rel * 16 + lane] = part;
      }
      ring[s] = issue<FMT>(S, ng, total, next, ic, ref[s], lane);
      QD_PIN_ISSUE();
    }
    if (ref[0].g >= ng) break;     // slot 0 was refilled first: nothing left for later slots
  }
  settle_to(ng);
}

// ---- control wave ----------------------------------------------------------

__device__ __forceinline__ void wait_stores() { asm volatile("s_waitcnt vmcnt(0)" ::: "memory"); }

__device__ __forceinline__ unsigned long long stamp(const PlanArgs& p, int g) {
  return p.epoch * (unsigned long long)p.ngroups + (unsigned long long)(g + 1);
}

// Stage a group's activation vector (and, for int4, its 16-value run sums) in
// LDS.  All loads of a batch are issued before any is consumed, so staging
// costs about one memory round trip per 8 KiB.
template <int FMT>
__device__ void stage_group_x(const Sched& S, int g, int lane, half_t* xs, float* xsum) {
  constexpr int kBatch = 8;
  const int Kp = S.J(g) * kSuperK;
  const __amdgpu_buffer_rsrc_t rx = make_rsrc(S.x(g), (uint32_t)(S.k(g) * 2));
  for (int i0 = 0; i0 < Kp; i0 += 64 * 8 * kBatch) {
    u32x4 v[kBatch];
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + (b * 64 + lane) * 8;
      v[b] = bload16_coherent(rx, (uint32_t)min(i, Kp) * 2);   // past K: zeros
    }
#pragma unroll
    for (int b = 0; b < kBatch; ++b) {
      const int i = i0 + (b * 64 + lane) * 8;
      float sum = 0.0f;
      if (FMT == QD_FMT_INT4_G64) {
        const half8_t h = __builtin_bit_cast(half8_t, v[b]);
#pragma unroll
        for (int e = 0; e < 8; ++e) sum += (float)h[e];
        sum += __shfl_xor(sum, 1);        // lanes 2q, 2q+1 hold one 16-value run
      }
      if (i < Kp) {
        *reinterpret_cast<u32x4*>(xs + i) = v[b];
        if (FMT == QD_FMT_INT4_G64 && (lane & 1) == 0) {
          const int t = i >> 4, jj = t >> 4, within = t & 15;
          xsum[16 * jj + 4 * (within & 3) + (within >> 2)] = sum;
        }
      }
    }
  }
}

// Row-group rg of group g may belong to a different member in each lane, so
// the member lookup uses per-lane reads.
__device__ __forceinline__ void store_row(const Sched& S, int g, int rg, int row, float v) {
  int mi = S.mem0(g);
  const int last = mi + S.nmem(g) - 1;
  while (mi < last && rg >= S.rg_begin_l(mi + 1)) ++mi;
  const int64_t n = (int64_t)(rg - S.rg_begin_l(mi)) * kTileRows + row;
  if (n < S.n_l(mi))
    __hip_atomic_store(S.y_l(mi) + n, __builtin_bit_cast(uint16_t, (half_t)v), __ATOMIC_RELAXED,
                       __HIP_MEMORY_SCOPE_AGENT);
}

// Reduce the compute waves' partials of group g, write finished rows, and
// combine row-groups split across workgroups.  A split row-group's partial
// travels as one 8-byte word per row holding the partial and the group's
// stamp, so it needs no separate flag: the last contributor of the row-group
// polls the others' words until every stamp is current, then adds them in
// workgroup order (deterministic) to its own partial and writes the rows.
__device__ void finish_group(const PlanArgs& p, const Sched& S, int g, int w, int lane,
                             const float* red) {
  const int a = S.a(g), b = S.b(g);
  if (a >= b) return;
  const int J = S.J(g);
  const int rg0 = a / J, nseg = (b - 1) / J - rg0 + 1;
  const int row = lane & 15;
  const bool first_split = (a != rg0 * J) || (b < (rg0 + 1) * J);
  const int rgl = rg0 + nseg - 1;
  const bool last_split = nseg > 1 && (b != (rgl + 1) * J);
  const uint32_t st = (uint32_t)stamp(p, g);
  float own[2] = {0.0f, 0.0f};                 // this workgroup's partials of split row-groups
  for (int s0 = 0; s0 < nseg; s0 += 4) {
    const int s = s0 + (lane >> 4);
    float sum = 0.0f;
    bool split = false;
    if (s < nseg) {
      // Tiles of row-group rg0 + s inside [a, b), summed in tile order.
      const int rg = rg0 + s;
      const int r0 = max(a, rg * J) - rg0 * J, r1 = min(b, (rg + 1) * J) - rg0 * J;
      for (int r = r0; r < r1; ++r) sum += red[r * 16 + row];
      split = (s == 0 && first_split) || (s == nseg - 1 && s > 0 && last_split);
      if (!split) store_row(S, g, rg, row, sum);
    }
    // Bring the split partials (lanes 0..15 for the first segment, the lanes
    // of segment nseg-1 for the last) to lanes 0..15.
    if (s0 == 0) own[0] = first_split ? sum : 0.0f;
    const int last_lane0 = ((nseg - 1) - s0) * 16;
    if (last_split && last_lane0 >= 0 && last_lane0 < 64) own[1] = __shfl(sum, last_lane0 + row);
  }
  const PSched* ms = S.s + g;
  for (int side = 0; side < 2; ++side) {
    if (side == 0 ? !first_split : !last_split) continue;
    const int wf = uni(side == 0 ? ms->wf0 : ms->wf1), nc = uni(side == 0 ? ms->nc0 : ms->nc1);
    const int wl = wf + nc - 1;
    const int rg = side == 0 ? rg0 : rgl;
    if (w != wl) {
      // Hand the partial to the last contributor.
      if (lane < 16) {
        const unsigned long long word =
            ((unsigned long long)st << 32) | __builtin_bit_cast(uint32_t, own[side]);
        __hip_atomic_store(p.slots + ((size_t)w * 2 + side) * 16 + row, word, __ATOMIC_RELAXED,
                           __HIP_MEMORY_SCOPE_AGENT);
      }
      continue;
    }
    float sum = 0.0f;
    for (int c = wf; c < wl; ++c) {
      const int ca = p.sched[(size_t)g * p.G + c].a;        // contributor's first tile
      const int cside = (rg == ca / J) ? 0 : 1;
      const unsigned long long* src = p.slots + ((size_t)c * 2 + cside) * 16 + row;
      unsigned long long word = 0;
      uint32_t spins = 0;
      for (;;) {
        word = __hip_atomic_load(src, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
        const bool ready = (uint32_t)(word >> 32) == st || lane >= 16;
        if (__ballot(!ready) == 0ull) break;
        if (++spins > kSpinLimit ||
            __hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) {
          if (lane == 0) atomicOr(p.err, 1u);
          break;
        }
      }
      sum += __builtin_bit_cast(float, (uint32_t)word);
    }
    sum += own[side];
    if (lane < 16) store_row(S, g, rg, row, sum);
  }
}

// Publish that this workgroup has finished every row it owes group g.
__device__ __forceinline__ void publish(const PlanArgs& p, int g, int w, int lane) {
  wait_stores();                                            // outputs before the stamp
  if (lane == 0)
    __hip_atomic_store(&p.flags[w], stamp(p, g), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
}

// Wait until every workgroup has published group g (one coherent read of all
// stamps per poll).
__device__ void wait_group(const PlanArgs& p, int g, int lane) {
  if (__hip_atomic_load(p.err, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT) != 0u) return;
  const unsigned long long target = stamp(p, g);
  const __amdgpu_buffer_rsrc_t rf = make_rsrc(p.flags, (uint32_t)p.G * 8);
  uint32_t spins = 0;
  for (;;) {
    bool ok = true;
    for (int base = 0; base < p.G; base += 128) {           // 2 stamps per lane per load
      const int i = base + 2 * lane;
      const u32x4 v = bload16_coherent(rf, (uint32_t)i * 8);
      const unsigned long long s0 = ((unsigned long long)v[1] << 32) | v[0];
      const unsigned long long s1 = ((unsigned long long)v[3] << 32) | v[2];
      ok = ok && (i >= p.G || s0 >= target) && (i + 1 >= p.G || s1 >= target);
    }
    if (__ballot(!ok) == 0ull) break;
    if (++spins > kSpinLimit) {
      if (lane == 0) atomicOr(p.err, 1u);
      break;
    }
  }
  asm volatile("" ::: "memory");
}

template <int FMT>
__device__ void control_wave(const PlanArgs& p, const Sched& S, int w, int lane, half_t* xs,
                             float* xsum, float* red) {
  // The control wave is on every group's critical path: let it issue ahead of
  // the compute waves that share its SIMD.
  __builtin_amdgcn_s_setprio(3);
  stage_group_x<FMT>(S, 0, lane, xs, xsum);
  for (int g = 0; g < p.ngroups; ++g) {
    wg_barrier();                 // activations of g staged
    wg_barrier();                 // compute waves finished g
    finish_group(p, S, g, w, lane, red);
    publish(p, g, w, lane);
    if (g + 1 < p.ngroups) {
      wait_group(p, g, lane);
      stage_group_x<FMT>(S, g + 1, lane, xs, xsum);
    }
  }
}

template <int FMT, int D>
__global__ __launch_bounds__(kWaves * 64) void stack_kernel(PlanArgs p) {
  extern __shared__ __attribute__((aligned(16))) uint8_t smem[];
  half_t* xs = reinterpret_cast<half_t*>(smem);
  float* xsum = reinterpret_cast<float*>(smem + p.x_bytes);
  float* red = reinterpret_cast<float*>(smem + p.x_bytes + p.xsum_bytes);
  uint8_t* tab = smem + p.x_bytes + p.xsum_bytes + p.red_bytes;
  uint32_t* next = reinterpret_cast<uint32_t*>(tab + p.tab_bytes);   // tile hand-out counter
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
    const int ng16 = p.ngroups * 2, nm16 = p.nmem * 2;     // 16-byte units
    for (int i = threadIdx.x; i < ng16 + nm16 + ng16; i += kWaves * 64) {
      u32x4 val;
      if (i < ng16) val = gsrc[i];
      else if (i < ng16 + nm16) val = msrc[i - ng16];
      else {
        const int q = i - ng16 - nm16, gi = q >> 1, half = q & 1;
        val = reinterpret_cast<const u32x4*>(p.sched + (size_t)gi * p.G + w)[half];
      }
      dst[i] = val;
    }
    if (threadIdx.x == 0) *next = 0u;
  }
  __syncthreads();

  if (wave == kCtl) {
    control_wave<FMT>(p, S, w, lane, xs, xsum, red);
  } else {
    const int last = p.ngroups - 1;
    const int total = S.off(last) + S.b(last) - S.a(last);
    compute_wave<FMT, D>(p, S, total, next, lane, xs, xsum, red);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

constexpr int kRing8 = 3;
constexpr int kRing4 = 4;

}  // namespace

}  // namespace qd

// ---------------------------------------------------------------------------
// Plan object

struct qd_stack_plan {
  int device = 0;
  bool persistent = false;
  int fmt = 0;
  std::vector<qd::StackGroup> replay;    // launch-per-group fallback (m > 1, K = 0, mixed formats)
  void* tables = nullptr;
  void* scratch = nullptr;
  size_t scratch_bytes = 0;
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
  int R;
};

size_t align_up(size_t v, size_t a) { return (v + a - 1) / a * a; }

const void* kernel_ptr(int fmt) {
  return fmt == QD_FMT_INT8_B32
             ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, kRing8>)
             : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT4_G64, kRing4>);
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

  // Persistent walker: one token row, one format, no empty-K groups.
  std::vector<HostGroup> groups;
  bool ok = (m == 1);
  int fmt = 0;
  for (int64_t i = 0; ok && i < n_ops;) {
    int64_t e = i + 1;
    while (e < n_ops && ops[e].group == ops[i].group) ++e;
    HostGroup hg{ops[i].x, ops[i].w.k, (int)ceil_div(ops[i].w.k, kSuperK), {}, 0};
    for (int64_t q = i; q < e; ++q) {
      if (ops[q].w.n == 0) continue;
      if (ops[q].w.k == 0) ok = false;
      if (fmt == 0) fmt = ops[q].w.fmt;
      if (ops[q].w.fmt != fmt) ok = false;
      hg.mem.push_back(PMember{static_cast<const uint8_t*>(ops[q].w.data), ops[q].y, ops[q].w.n,
                               hg.R, 0});
      hg.R += (int)ceil_div(ops[q].w.n, kTileRows);
    }
    if (!hg.mem.empty()) groups.push_back(std::move(hg));
    i = e;
  }
  int cus = 0;
  if (ok && !groups.empty()) {
    if (hipDeviceGetAttribute(&cus, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess ||
        cus <= 0)
      ok = false;
  } else {
    ok = false;
  }
  if (!ok) {
    plan->replay = std::move(replay);
    *out = plan;
    return QD_OK;
  }

  const int G = cus;
  const int ng = (int)groups.size();
  std::vector<PGroup> pg(ng);
  std::vector<PMember> pm;
  std::vector<PSched> ps((size_t)ng * G);
  std::vector<int32_t> off(G, 0);
  int maxJ = 1, maxRel = 1;
  std::vector<int64_t> s(G + 1);
  for (int g = 0; g < ng; ++g) {
    HostGroup& hg = groups[g];
    const int64_t J = hg.J, R = hg.R, T = R * J;
    if (T > (int64_t)INT32_MAX / 2) {
      delete plan;
      return QD_ESHAPE;
    }
    pg[g] = PGroup{hg.x, hg.k, hg.J, hg.R, (int32_t)pm.size(), (int32_t)hg.mem.size()};
    for (const PMember& mm : hg.mem) pm.push_back(mm);
    maxJ = std::max(maxJ, hg.J);
    // Tile ranges per workgroup: whole row-groups when that splits the group
    // evenly to within 5% (no cross-workgroup combine), else an even split of
    // tiles.
    if (R >= G && (R + G - 1) / G * G * 20 <= R * 21) {
      for (int w = 0; w <= G; ++w) s[w] = (int64_t)w * R / G * J;
    } else {
      const int64_t Gg = std::min<int64_t>(G, T);
      for (int w = 0; w <= G; ++w) s[w] = w <= Gg ? (int64_t)w * T / Gg : T;
    }
    auto owner = [&](int64_t t) {   // workgroup whose (non-empty) range holds tile t
      int lo = 0, hi = G - 1;
      while (lo < hi) {
        const int mid = (lo + hi + 1) / 2;
        if (s[mid] <= t) lo = mid;
        else hi = mid - 1;
      }
      return lo;
    };
    for (int w = 0; w < G; ++w) {
      PSched& e = ps[(size_t)g * G + w];
      const int64_t a = s[w], b = s[w + 1];
      e = PSched{(int32_t)a, (int32_t)b, 0, 1, 0, 1, off[w], (int32_t)(a / J)};
      if (a >= b) continue;
      off[w] += (int32_t)(b - a);
      const int64_t rg0 = a / J, rgl = (b - 1) / J;
      maxRel = std::max<int>(maxRel, (int)(b - rg0 * J));
      const int f0 = owner(rg0 * J), l0 = owner(rg0 * J + J - 1);
      const int f1 = owner(rgl * J), l1 = owner(rgl * J + J - 1);
      e.wf0 = f0;
      e.nc0 = l0 - f0 + 1;
      e.wf1 = f1;
      e.nc1 = l1 - f1 + 1;
    }
  }
  const size_t x_bytes = align_up((size_t)maxJ * kSuperK * 2, 16);
  const size_t xsum_bytes = fmt == QD_FMT_INT4_G64 ? align_up((size_t)maxJ * 16 * 4, 16) : 0;
  const size_t red_bytes = align_up((size_t)maxRel * 16 * 4, 16);
  const size_t tab_bytes = (size_t)ng * sizeof(PGroup) + pm.size() * sizeof(PMember) +
                           (size_t)ng * sizeof(PSched);
  const size_t lds = x_bytes + xsum_bytes + red_bytes + tab_bytes + 16;
  hipDeviceProp_t prop;
  if (hipGetDeviceProperties(&prop, dev) != hipSuccess) {
    delete plan;
    return QD_EDEVICE;
  }
  const void* kfn = kernel_ptr(fmt);
  const size_t lds_max = std::max<size_t>(prop.sharedMemPerBlock, prop.maxSharedMemoryPerMultiProcessor);
  if (lds > lds_max) {
    delete plan;
    return QD_ESHAPE;
  }
  if (lds > 65536 &&
      hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)lds) != hipSuccess) {
    delete plan;
    return QD_ESHAPE;
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, kWaves * 64, lds) != hipSuccess ||
      per_cu < 1) {
    delete plan;
    return QD_ESHAPE;
  }

  // Device tables, then scratch.
  const size_t o_groups = 0;
  const size_t o_mem = align_up(o_groups + sizeof(PGroup) * ng, 256);
  const size_t o_sched = align_up(o_mem + sizeof(PMember) * pm.size(), 256);
  const size_t t_bytes = align_up(o_sched + sizeof(PSched) * ps.size(), 256);
  const size_t s_flags = 0;
  const size_t s_slots = align_up(sizeof(unsigned long long) * G, 256);
  const size_t s_err = align_up(s_slots + sizeof(unsigned long long) * G * 2 * 16, 256);
  const size_t s_bytes = s_err + 256;
  std::vector<uint8_t> host(t_bytes, 0);
  memcpy(host.data() + o_groups, pg.data(), sizeof(PGroup) * ng);
  memcpy(host.data() + o_mem, pm.data(), sizeof(PMember) * pm.size());
  memcpy(host.data() + o_sched, ps.data(), sizeof(PSched) * ps.size());
  if (hipMalloc(&plan->tables, t_bytes) != hipSuccess ||
      hipMalloc(&plan->scratch, s_bytes) != hipSuccess ||
      hipMemcpy(plan->tables, host.data(), t_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipMemset(plan->scratch, 0, s_bytes) != hipSuccess || hipDeviceSynchronize() != hipSuccess) {
    if (plan->tables) (void)hipFree(plan->tables);
    if (plan->scratch) (void)hipFree(plan->scratch);
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
  a.slots = reinterpret_cast<unsigned long long*>(sb + s_slots);
  a.err = reinterpret_cast<uint32_t*>(sb + s_err);
  a.ngroups = ng;
  a.nmem = (int32_t)pm.size();
  a.G = G;
  a.x_bytes = (int32_t)x_bytes;
  a.xsum_bytes = (int32_t)xsum_bytes;
  a.red_bytes = (int32_t)red_bytes;
  a.tab_bytes = (int32_t)tab_bytes;
  plan->scratch_bytes = s_bytes;
  plan->lds = lds;
  plan->fmt = fmt;
  plan->persistent = true;
  *out = plan;
  return QD_OK;
}

qd_status plan_run(qd_stack_plan* plan, hipStream_t s) {
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess || dev != plan->device) return QD_EDEVICE;
  if (!plan->persistent) return launch_groups(plan->replay, s) == hipSuccess ? QD_OK : QD_ELAUNCH;
  plan->args.epoch = ++plan->epoch;
  void* kargs[] = {&plan->args};
  const hipError_t e = hipLaunchCooperativeKernel(kernel_ptr(plan->fmt), dim3(plan->args.G),
                                                  dim3(kWaves * 64), kargs, (unsigned)plan->lds, s);
  if (e != hipSuccess) {
    --plan->epoch;
    return QD_ELAUNCH;
  }
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

void plan_destroy(qd_stack_plan* plan) {
  if (!plan) return;
  if (plan->tables) (void)hipFree(plan->tables);
  if (plan->scratch) (void)hipFree(plan->scratch);
  delete plan;
}

}  // namespace qd
