// Persistent decode-step kernel: one launch walks every group of the step.
//
// Decode streams every quantized weight once per token (Qwen3-VL 4B/8B Core
// AI cards, Measured paragraph), so a step's time is the weight stream plus
// whatever stalls it.  Per-group launches stall it at every group boundary:
// the next kernel starts loading only after the previous one drains.  Here the
// weight stream keeps going across group boundaries:
//
//   * one workgroup per CU (all co-resident), 16 waves:
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
//     published it, and releases the compute waves (one workgroup barrier
//     per group), so an op may consume an earlier op's output;
//   * a group that depends on no earlier group (reads nothing one writes,
//     writes nothing one reads or writes) skips that device-wide wait; a
//     bound on how far the workgroups may drift apart is kept instead (a
//     wait, overlapped with the streaming, for the group a plan-chosen lag
//     before);
//   * one token row: the control wave stages each group's activation vector
//     (and, with glue, gamma or the gated product's second block) straight
//     into LDS and applies the prologue there;
//   * up to 16 token rows: compute waves read the activation blocks
//     themselves, from copies in matrix-core order where the plan keeps them
//     (made before the step, or written by the op producing them), and the
//     partials are 16 x 16 per tile; groups too large for the partials in
//     LDS are split into row ranges that need no device-wide wait between
//     them; with glue, RMSNorm is applied to each block from per-token
//     factors the producing op's workgroups prepare (sum-of-squares
//     records), and a gate|up group run paired writes the gated product
//     into the copy its consumer reads;
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
#include <tuple>
#include <mutex>
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
  kNoWait = 4,          // no device-wide wait at the boundary: a further row range of the op(s)
                        // before, or a group independent of every earlier group
  kCleanLines = 8,      // x is written earlier in the step, but no cache can hold a stale copy of its
                        // lines: after the barrier it is read through the caches
  kPaired = 16,         // several token rows: a two-member group whose row-group i of both members
                        // forms one unit (virtual row-group 2i + b is member b's row-group i); it
                        // writes the gated product of its two outputs for a later group
  kIndependent = 32,    // independent of every earlier group (with kNoWait): at most the plan's
                        // lag bounds how far the workgroups drift apart (see control_wave)
  kDynamic = 64,        // one token row, the last group: its row-groups are not split in advance;
                        // workgroups claim them a chunk at a time as they get there (see
                        // finish_dynamic)
};

struct PGroup {         // 64 bytes
  const uint16_t* x;
  const uint16_t* gamma;  // RMSNorm weight (prologue QD_PRO_RMSNORM)
  const uint16_t* xt;     // m > 1: x in matrix-core order (plan scratch), or null; under the
                          // gated product it holds the product itself
  int32_t k;
  int32_t J;            // super-blocks per row
  int32_t R;            // row-groups in the group
  int32_t mem0;         // first member in the member table
  int32_t n_mem;
  int32_t pro;          // qd_prologue of the group's input
  float eps;
  int32_t order;        // kStageEarly | kAckOutputs | kNoWait | kCleanLines | kPaired
  int32_t ss0;          // m > 1 under RMSNorm: first sum-of-squares record of x
  int32_t ss_n;         // and the number of records that add up to it
};

struct PMember {        // 48 bytes
  const uint8_t* blob;
  uint16_t* y;
  int64_t n;
  int32_t rg_begin;     // first row-group of this member within its group
  int32_t epi;          // qd_epilogue of this member's outputs
  int32_t ld;           // elements between token rows of y (m > 1)
  int32_t ss;           // m > 1: first of the G sum-of-squares records of these outputs (record
                        // ss + w from workgroup w), or -1
  uint16_t* yt;         // m > 1: where the outputs also go in matrix-core order, or null (in a
                        // paired group, the first member's is where the gated product goes)
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
  float* ss;                  // m > 1: sum-of-squares records, 16 floats (one per token row) each
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
  int32_t lag;                // before an independent group: how many groups behind may the slowest
                              // workgroup be (0: unbounded); see control_wave
  // The dynamic last group (kDynamic), if dyn_c > 0: chunks of dyn_c row-groups are claimed
  // from dyn_ctr[epoch & 1] (the other counter is cleared for the next run); dyn_nch chunks in
  // all, at most dyn_max per workgroup, dyn_q claimed ahead of the tile hand-out; partial
  // slots and row-group counts reused modulo dyn_rcap and dyn_scap (powers of two).
  uint32_t* dyn_ctr;
  int32_t dyn_c;
  int32_t dyn_q;
  int32_t dyn_nch;
  int32_t dyn_max;
  int32_t dyn_rcap;
  int32_t dyn_scap;
  int32_t dyn_win;            // row-groups compute waves may run ahead of the reduction
  int32_t defer;              // a dynamic last group and 6 GiB of weights or more: stores may follow the staging
};

template <int FMT> struct Fmt;
template <> struct Fmt<QD_FMT_INT8_B32> {
  using Tile = Tile8;
  static constexpr int kT = kTileBytes8;
  __device__ static Tile load(__amdgpu_buffer_rsrc_t r, int lane, int j = 0) { return load_tile8(r, j, lane); }
};
template <> struct Fmt<QD_FMT_INT4_G64> {
  using Tile = Tile4;
  static constexpr int kT = kTileBytes4;
  __device__ static Tile load(__amdgpu_buffer_rsrc_t r, int lane, int j = 0) { return load_tile4(r, j, lane); }
};

// At one token row a hand-out covers ku1(fmt) consecutive super-blocks of one
// row-group (consecutive tiles in the blob).  INT4 tiles are half the bytes
// of int8 ones for the same hand-out work (the LDS counter, the address
// arithmetic, one partial, one count): two per hand-out put INT4 at about
// int8's bytes per hand-out.  A row-group's last hand-out may hold fewer.
#ifndef QD_PLAN_KU4
#define QD_PLAN_KU4 2
#endif
__host__ __device__ constexpr int ku1(int fmt) { return fmt == QD_FMT_INT4_G64 ? QD_PLAN_KU4 : 1; }

template <int FMT, int KU> struct KTiles {
  typename Fmt<FMT>::Tile t[KU];
};
template <bool C, typename A, typename B> struct Pick { using type = A; };
template <typename A, typename B> struct Pick<false, A, B> { using type = B; };
// What one hand-out at one token row loads.
template <int FMT>
using Hand1 = typename Pick<ku1(FMT) == 1, typename Fmt<FMT>::Tile, KTiles<FMT, ku1(FMT)>>::type;

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

// A workgroup's claims on the dynamic last group, in LDS (after the tile
// counter and the flags).  The control wave appends chunk ids in claim order;
// compute waves map their hand-outs in the group onto them.
struct DynCtl {
  int32_t claimed;      // chunks held (valid entries of chunk[])
  int32_t ended;        // no further chunk for this workgroup (the group is used up, or the cap)
  int32_t reduced;      // the group's row-groups reduced so far, in this workgroup's order
  int32_t pad;
  int32_t chunk[1];     // [dyn_max]
};

// The workgroup's schedule, resident in LDS.  Reads are wave-uniform.
struct Sched {
  const PGroup* g;
  const PMember* m;
  const PSched* s;
  // The dynamic last group (dyn_c > 0): claims, partial-slot and count masks,
  // and the row-groups compute waves may run ahead of the reduction.
  DynCtl* dyn;
  int dyn_c, dyn_rmask, dyn_smask, dyn_win;
  uint32_t spin;
  uint32_t* err;
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
  __device__ int64_t k(int gi) const { return (int64_t)uni(g[gi].k); }
  __device__ int ss0(int gi) const { return uni(g[gi].ss0); }
  __device__ int ss_n(int gi) const { return uni(g[gi].ss_n); }
  __device__ bool paired(int gi) const { return (order(gi) & kPaired) != 0; }
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
  __device__ int64_t ld(int mi) const { return (int64_t)uni(m[mi].ld); }
  __device__ int epi(int mi) const { return uni(m[mi].epi); }
  __device__ int ss(int mi) const { return uni(m[mi].ss); }
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
  int lseg;   // the dynamic group: row-group in this workgroup's claim order (rel and seg
              // are then that modulo the slot and count capacities); else -1
};

struct IssueCursor {
  int g;                // current group (-1 before the first)
  int off_next;         // sequence index where the next group starts
  int u, seg, j;        // last issued tile (or unit): index within the workgroup's part,
                        // (segment, super-block); for units seg counts units, and at one
                        // token row j counts hand-outs of ku1 super-blocks
  int J, rg0, nseg;
  int mem, mem_last;
  bool paired;          // the current group is paired (kPaired)
};

template <int FMT>
__device__ __forceinline__ Hand1<FMT> issue(const Sched& S, int ngroups, int total,
                                            uint32_t* next, IssueCursor& c,
                                            TileRef& ref, int lane, bool take = true) {
  constexpr int T = Fmt<FMT>::kT;
  constexpr int KU = ku1(FMT);
  // take == false: claim nothing; the load below then reads an empty buffer
  // (zeros, no memory traffic), which keeps the caller's control flow uniform.
  uint32_t got = (uint32_t)total;
  if (take && lane == 0) got = atomicAdd(next, 1u);
  const int idx = uni((int)got);
  const uint8_t* base = nullptr;
  uint32_t nbytes = 0;
  ref.g = ngroups;
  ref.lseg = -1;
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
    const int Ju = (c.J + KU - 1) / KU;                 // hand-outs per row-group
    if (S.dyn_c > 0 && c.g == ngroups - 1) {
      // The dynamic last group: hand-out u is hand-out t of the k-th chunk
      // this workgroup claimed (the control wave claims ahead of the
      // hand-outs; it never reuses an entry).
      // (The cursor moves forward by the hand-outs since the wave's last one,
      // as in a fixed range: c.seg counts chunks, c.j hand-outs within one.)
      const int per = S.dyn_c * Ju;
      c.j += u - c.u;
      c.u = u;
      while (c.j >= per) {
        c.j -= per;
        ++c.seg;
      }
      const int k = c.seg;
      int jh = c.j, sq = 0;
      while (jh >= Ju) {
        jh -= Ju;
        ++sq;
      }
      int ch = -1;
      for (uint32_t spins = 0;; ++spins) {
        const bool ended = lds_get(&S.dyn->ended) != 0;
        if (k < lds_get(&S.dyn->claimed)) {
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
          ch = uni(S.dyn->chunk[k]);
          break;
        }
        if (ended) break;                             // no chunk k: the sequence ends here
        if (spins > S.spin) {
          if (lane == 0) atomicOr(S.err, 2u);
          break;
        }
        __builtin_amdgcn_s_sleep(1);
      }
      if (ch >= 0) {
        const int lseg = k * S.dyn_c + sq;
        const int rg = ch * S.dyn_c + sq;            // past the group (its last chunk): zeros
        const int j0 = jh * KU;
        const int nv = min(KU, c.J - j0);
        if (rg < S.R(c.g)) {
          int mi = c.mem;                             // members in row-group order; any may hold rg
          while (mi < c.mem_last && rg >= S.rg_begin(mi + 1)) ++mi;
          base = S.blob(mi) + ((int64_t)(rg - S.rg_begin(mi)) * c.J + j0) * T;
          nbytes = (uint32_t)(nv * T);
        }
        ref.g = c.g;
        ref.j = j0;
        ref.rel = u & S.dyn_rmask;
        ref.seg = lseg & S.dyn_smask;
        ref.nv = nv;
        ref.lseg = lseg;
      }
      const __amdgpu_buffer_rsrc_t rd = make_rsrc(base, nbytes);
      if constexpr (KU == 1) {
        return Fmt<FMT>::load(rd, lane);
      } else {
        KTiles<FMT, KU> t2;
#pragma unroll
        for (int q = 0; q < KU; ++q) t2.t[q] = Fmt<FMT>::load(rd, lane, q);
        return t2;
      }
    }
    c.j += u - c.u;
    c.u = u;
    while (c.j >= Ju) {
      c.j -= Ju;
      ++c.seg;
    }
    const int rg = c.rg0 + c.seg;
    while (c.mem < c.mem_last && rg >= S.rg_begin(c.mem + 1)) ++c.mem;
    const int j0 = c.j * KU;
    const int nv = min(KU, c.J - j0);
    base = S.blob(c.mem) + ((int64_t)(rg - S.rg_begin(c.mem)) * c.J + j0) * T;
    nbytes = (uint32_t)(nv * T);                        // a missing last tile reads as zeros
    ref.g = c.g;
    ref.j = j0;
    ref.rel = u;
    ref.seg = c.seg;
    ref.nv = nv;
  }
  const __amdgpu_buffer_rsrc_t r = make_rsrc(base, nbytes);
  if constexpr (KU == 1) {
    return Fmt<FMT>::load(r, lane);
  } else {
    KTiles<FMT, KU> t;
#pragma unroll
    for (int q = 0; q < KU; ++q) t.t[q] = Fmt<FMT>::load(r, lane, q);
    return t;
  }
}

// Up to 16 token rows: the sequence is made of units, U row-groups at one
// super-block (unit-row major: units (q, 0), (q, 1), ... (q, J - 1), then
// q + 1), so that one activation block serves U tiles.  The last unit of a
// range may hold fewer row-groups; its missing tiles read as zeros.  In a
// paired group (PAIR instances only) row-group v is row-group v / 2 of
// member v % 2, so a unit of two holds the same rows of both members.
template <int FMT, int U>
struct Unit {
  typename Fmt<FMT>::Tile w[U];
};

template <int FMT, int U, bool PAIR>
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
  ref.lseg = -1;
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
      c.paired = PAIR && S.paired(c.g);
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
    if (PAIR && c.paired) {
#pragma unroll
      for (int q = 0; q < U; ++q) {
        if (q < nv) {
          const int rg = c.rg0 + seg0 + q;
          base[q] = S.blob(c.mem + (rg & 1)) + ((int64_t)(rg >> 1) * c.J + c.j) * T;
          nbytes[q] = T;
        }
      }
    } else {
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

// INT4 g64 at one token row on the matrix cores.  The codes become fp16
// subnormals with one AND per pair, as in the GEMV: for a word whose nibble p
// holds code (0,2,4,6,1,3,5,7)[p], w & 0x000F000F and (w >> 8) & 0x000F000F
// are codes (0,1) and (4,5) times 2^-24, w & 0x00F000F0 and
// (w >> 8) & 0x00F000F0 codes (2,3) and (6,7) times 2^-20.  Per group of 64
// codes, one 16x16x32 product takes the lane's eight 2^-24 codes (from its two
// words) and another the eight 2^-20 ones, each against the matching x pairs;
// the matrix core also sums the group's four K quarters, which the VALU dot
// products left to a cross-lane reduction.  With the same x in every A row,
// every output row of the product is the weight row's dot product, so lane
// (g, rho) ends with row rho's total.  The group's activation sum X comes
// from the same two x operands against an all-ones B (every output is the sum
// over the group), so nothing beyond x itself is staged.  Products are exact
// (a 4-bit code times an fp16 value, scaled by a power of two) and sums are
// fp32, as in the GEMV; y = 2^24 sum_a s_a (lo_a + hi_a / 16) + sum_a min_a X_a.
// (Measured against group sums added up by the control wave as it stages x,
// wall us per step on three devices: 8B INT4 762 -> 722-724, 762-764 ->
// 736-738, 765 -> 753-757; that staging is on every boundary's critical
// path.)
__device__ __forceinline__ float tile_row4(const Tile4& T, const half_t* xs_j, int g) {
  const half8_t mt = __builtin_bit_cast(half8_t, T.meta);
  const uint32_t m = 0x000F000Fu, m4 = 0x00F000F0u;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  const half_t one = (half_t)1.0f;
  const half8_t ones = {one, one, one, one, one, one, one, one};
  float acc_s = 0.0f, acc = 0.0f;
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int s = a >> 1, h = a & 1;
    // x pairs (0,1), (4,5), (8,9), (12,13) of the lane's 16 values against
    // the 2^-24 codes, (2,3), (6,7), (10,11), (14,15) against the 2^-20 ones:
    // read as dword pairs two apart, straight into operand order (the empty
    // asm keeps the two halves from being merged into contiguous loads that
    // would then need register moves).
    const uint32_t* x32 = reinterpret_cast<const uint32_t*>(xs_j + 64 * a + 16 * g);
    const u32x4 alo = {x32[0], x32[2], x32[4], x32[6]};
    asm volatile("" ::: "memory");
    const u32x4 ahi = {x32[1], x32[3], x32[5], x32[7]};
    const uint32_t w0 = T.c[s][2 * h], w1 = T.c[s][2 * h + 1];
    const uint32_t w08 = w0 >> 8, w18 = w1 >> 8;
    const u32x4 blo = {w0 & m, w08 & m, w1 & m, w18 & m};
    const u32x4 bhi = {w0 & m4, w08 & m4, w1 & m4, w18 & m4};
    const float4_t lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(half8_t, alo), __builtin_bit_cast(half8_t, blo), zero, 0, 0, 0);
    const float4_t hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(half8_t, ahi), __builtin_bit_cast(half8_t, bhi), zero, 0, 0, 0);
    float4_t xsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, alo), ones, zero, 0, 0, 0);
    xsum = __builtin_amdgcn_mfma_f32_16x16x32_f16(__builtin_bit_cast(half8_t, ahi), ones, xsum, 0, 0, 0);
    acc_s = __builtin_fmaf((float)mt[a], __builtin_fmaf(hi[0], 0.0625f, lo[0]), acc_s);
    acc = __builtin_fmaf((float)mt[4 + a], xsum[0], acc);
  }
  return __builtin_fmaf(acc_s, 16777216.0f, acc);
}

// One tile at one token row: lanes 0..15 get the 16 rows' sums (INT4: every
// lane gets its row's).
template <int FMT>
__device__ __forceinline__ float tile_row(const typename Fmt<FMT>::Tile& T, const half_t* xs, int j, int g);
template <>
__device__ __forceinline__ float tile_row<QD_FMT_INT8_B32>(const Tile8& T, const half_t* xs, int j, int g) {
  // Per 32-block one 16x16x32 product of the lane's 8 codes (exact fp16
  // integers) against its 8 activations; with the same x in every A row each
  // output row is the weight row's block sum, so lane (g, rho) gets row rho's.
  const half_t* xs_j = xs + j * kSuperK;
  const half8_t scales = __builtin_bit_cast(half8_t, T.sc);
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float acc = 0.0f;
#pragma unroll
  for (int s = 0; s < 4; ++s) {
#pragma unroll
    for (int h = 0; h < 2; ++h) {
      const half8_t xv = *reinterpret_cast<const half8_t*>(xs_j + 64 * s + 32 * h + 8 * g);
      const half8_t bq = codes_to_half8(T.c[s][2 * h], T.c[s][2 * h + 1]);
      const float4_t pr = __builtin_amdgcn_mfma_f32_16x16x32_f16(xv, bq, zero, 0, 0, 0);
      acc = __builtin_fmaf((float)scales[2 * s + h], pr[0], acc);
    }
  }
  return acc;
}
template <>
__device__ __forceinline__ float tile_row<QD_FMT_INT4_G64>(const Tile4& T, const half_t* xs, int j, int g) {
  return tile_row4(T, xs + j * kSuperK, g);
}

// Up to 16 token rows (MT = 16).  The activation block of super-block j,
// X[0..15][256 j .. 256 j + 255], as the eight A operands of the tile's
// 16x16x32 products: operand q of lane (gq, rho) holds 8 of token rho's
// values.
//   int8 b32: the 8 at K position kpos(q, gq) = 32 q + 8 gq within the
//             super-block (operand q = 32-block q).
//   INT4 g64: operands 2a, 2a + 1 cover the lane's 16 consecutive values of
//             group a, at 64 a + 16 gq: its halves start at kpos(2a, gq) and
//             kpos(2a + 1, gq) = kpos(2a, gq) + 8.  Operand 2a holds value
//             pairs 0, 2, 4, 6 of the 16 (against codes taken as 2^-24
//             subnormals) and operand 2a + 1 pairs 1, 3, 5, 7 (against codes
//             times 2^-20): int4_lo / int4_hi of the two halves.
template <int FMT>
__host__ __device__ constexpr int kpos(int q, int gq) {
  return FMT == QD_FMT_INT8_B32 ? 32 * q + 8 * gq : 64 * (q >> 1) + 16 * gq + 8 * (q & 1);
}
__device__ __forceinline__ u32x4 int4_lo(const u32x4& h0, const u32x4& h1) {
  return (u32x4){h0[0], h0[2], h1[0], h1[2]};
}
__device__ __forceinline__ u32x4 int4_hi(const u32x4& h0, const u32x4& h1) {
  return (u32x4){h0[1], h0[3], h1[1], h1[3]};
}
// The eight operands from the natural halves (INT4: in place).
template <int FMT>
__device__ __forceinline__ void to_operand_order(u32x4 (&xa)[8]) {
  if constexpr (FMT == QD_FMT_INT4_G64) {
#pragma unroll
    for (int a = 0; a < 4; ++a) {
      const u32x4 h0 = xa[2 * a], h1 = xa[2 * a + 1];
      xa[2 * a] = int4_lo(h0, h1);
      xa[2 * a + 1] = int4_hi(h0, h1);
    }
  }
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
  to_operand_order<FMT>(xa);
}

// Where output row n (of a K-long input row of a later group) goes in that
// group's matrix-core-ordered copy, token row t: the inverse of kpos.
template <int FMT>
__device__ __forceinline__ int64_t xt_index(int64_t n, int t) {
  const int64_t j = n >> 8;
  const int w = (int)(n & 255);
  // INT4: value r = w & 15 of the lane's run, pair (r & 7) / 2 of half r / 8
  // (see kpos): odd pairs go to operand 2a + 1; slot half * 2 + pair / 2.
  const int q = FMT == QD_FMT_INT8_B32 ? w >> 5 : 2 * (w >> 6) + ((w >> 1) & 1);
  const int gq = FMT == QD_FMT_INT8_B32 ? (w >> 3) & 3 : (w >> 4) & 3;
  const int pos = FMT == QD_FMT_INT8_B32 ? (w & 7) : ((w >> 3) & 1) * 4 + ((w >> 2) & 1) * 2 + (w & 1);
  return (((j * 8 + q) * 64 + gq * 16 + t) << 3) + pos;
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

// INT4 g64, per group a: the codes as fp16 subnormals with one AND per pair,
// as at one token row (nibble p of a word holds code (0,2,4,6,1,3,5,7)[p], so
// w & 0x000F000F and (w >> 8) & 0x000F000F are codes (0,1) and (4,5) times
// 2^-24, w & 0x00F000F0 and (w >> 8) & 0x00F000F0 codes (2,3) and (6,7) times
// 2^-20): one product per kind against the operand holding the matching value
// pairs (see kpos), sums in fp32 apart, sum(c x) = 2^24 (lo + hi / 16).  Then
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
  const uint32_t m = 0x000F000Fu, m4 = 0x00F000F0u;
  const float4_t zero = {0.0f, 0.0f, 0.0f, 0.0f};
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
#pragma unroll
  for (int a = 0; a < 4; ++a) {
    const int s = a >> 1, h = a & 1;
    const uint32_t w0 = T.c[s][2 * h], w1 = T.c[s][2 * h + 1];
    const uint32_t w08 = w0 >> 8, w18 = w1 >> 8;
    const u32x4 blo = {w0 & m, w08 & m, w1 & m, w18 & m};
    const u32x4 bhi = {w0 & m4, w08 & m4, w1 & m4, w18 & m4};
    const float4_t lo = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(half8_t, xa[2 * a]), __builtin_bit_cast(half8_t, blo), zero, 0, 0, 0);
    const float4_t hi = __builtin_amdgcn_mfma_f32_16x16x32_f16(
        __builtin_bit_cast(half8_t, xa[2 * a + 1]), __builtin_bit_cast(half8_t, bhi), zero, 0, 0, 0);
    const float sc = (float)mt[a] * 16777216.0f, mn = (float)mt[4 + a];
#pragma unroll
    for (int i = 0; i < 4; ++i)
      acc[i] = __builtin_fmaf(sc, __builtin_fmaf(hi[i], 0.0625f, lo[i]), __builtin_fmaf(mn, xs[a][i], acc[i]));
  }
  return acc;
}

// Up to 16 token rows under RMSNorm: the activation block as read (raw x)
// becomes u = fp16(gamma * fp16(x * r)), with the group's per-token factors r
// (lane (gq, rho) holds token rho) and gamma, both staged in LDS by the
// control wave before the group's barrier.  K positions past K hold x = 0
// and gamma = 0, so u = 0 there.
template <int FMT>
__device__ __forceinline__ void rms_block(u32x4 (&xa)[8], const half_t* gam, const float* rinv, int j,
                                          int lane) {
  const int gq = lane >> 4;
  const float r = rinv[lane & 15];
  u32x4 ga[8];
#pragma unroll
  for (int b = 0; b < 8; ++b) ga[b] = *reinterpret_cast<const u32x4*>(gam + j * kSuperK + kpos<FMT>(b, gq));
  to_operand_order<FMT>(ga);            // gamma in the activations' order
#pragma unroll
  for (int b = 0; b < 8; ++b) xa[b] = rms8(xa[b], r, ga[b]);
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
__device__ void prologue_share(const Sched& S, int g, int wave, int lane, half_t* xs, float* pf, int nrms);
template <int FMT, int MT, int U> struct RingOf { using type = Hand1<FMT>; };
template <int FMT, int U> struct RingOf<FMT, 16, U> { using type = Unit<FMT, U>; };

// At up to 16 token rows with glue (GLUE), xs holds the RMSNorm gamma of the
// current group and xsum its 16 per-token factors.
template <int FMT, int D, bool RESERVE, int R, int MT, int U, bool GLUE>
__device__ void compute_wave(const PlanArgs& p, const Sched& S, int total, uint32_t* next,
                             int lane, half_t* xs, float* xsum, float* red,
                             uint32_t* cnt, const int* stalled, const int* staged) {
  using Tile = typename RingOf<FMT, MT, U>::type;
  const int ng = p.ngroups;
  const int g4 = lane >> 4;
  IssueCursor ic{-1, 0, 0, 0, 0, 1, 0, 0, 0, 0, false};
  Tile ring[D];
  TileRef ref[D];
  auto next_tile = [&](TileRef& r, int ln, bool take = true) {
    if constexpr (MT == 1) return issue<FMT>(S, ng, total, next, ic, r, ln, take);
    else return issue_unit<FMT, U, GLUE>(S, ng, total, next, ic, r, ln, take);
  };
  // MT > 1: the unit's activation block is loaded when the unit is computed,
  // not with its tiles (measured on the 8B steps at 16 token rows, us: int8
  // 1810 -> 1734, INT4 1287 -> 1259 against loading it with the tiles when it
  // is already readable; the block is read from L2 and the unit's weights are
  // long in flight by then).  One block's registers serve every ring slot.
  u32x4 xr[8];
  int cg = -1;                      // last group whose activations this wave has waited for
  int nrms = 0;                     // RMSNorm prologues passed (one token row, glue)
  auto settle_to = [&](int g) {
    while (cg < g) {
      ++cg;
      if (cg >= ng) continue;
      if constexpr (GLUE && MT == 1) {
        if (S.pro(cg) != QD_PRO_NONE) {
          // This wave's share of the group's prologue pass, once the control
          // wave has staged the data (bounded wait; a timeout is reported).
          const int* flag = reinterpret_cast<const int*>(xsum) + 1;
          for (uint32_t spins = 0; lds_get(flag) < cg + 1; ++spins) {
            if (spins > S.spin) {
              if (lane == 0) atomicOr(S.err, 2u);
              break;
            }
            __builtin_amdgcn_s_sleep(1);
          }
          __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
          if (S.pro(cg) == QD_PRO_RMSNORM) ++nrms;
          prologue_share(S, cg, uni((int)(threadIdx.x >> 6)), lane, xs, xsum, nrms);
        }
      }
      wg_barrier();
    }
  };
  auto compute = [&](int s) {
    const Tile& t = ring[s];
    const TileRef& r = ref[s];
    settle_to(r.g);
    if constexpr (MT == 1) {
      float part;
      if constexpr (ku1(FMT) == 1) {
        part = tile_row<FMT>(t, xs, r.j, g4);
      } else {
        // The tiles' sums in tile order.  A missing last tile (J odd) holds
        // zero codes, scales and mins, and reads zero activations (the
        // staging's loads past x return zeros), so it adds exactly zero.
        part = tile_row<FMT>(t.t[0], xs, r.j, g4);
#pragma unroll
        for (int q = 1; q < ku1(FMT); ++q) part += tile_row<FMT>(t.t[q], xs, r.j + q, g4);
      }
      if (r.lseg >= 0) {
        // The dynamic group reuses partial slots and counts: row-group lseg
        // may start only when the row-group dyn_w before it is reduced.
        for (uint32_t spins = 0; r.lseg >= lds_get(&S.dyn->reduced) + S.dyn_win; ++spins) {
          if (spins > S.spin) {
            if (lane == 0) atomicOr(S.err, 2u);
            break;
          }
          __builtin_amdgcn_s_sleep(1);
        }
      }
      if (lane < 16) red[r.rel * 16 + lane] = part;
    } else {
      load_xblock<FMT>(S, r.g, r.j, p.m, lane, !(S.order(r.g) & (kStageEarly | kCleanLines)), xr);
      // (A gated product needs nothing here: the group's copy holds it.)
      if constexpr (GLUE)
        if (S.pro(r.g) == QD_PRO_RMSNORM) rms_block<FMT>(xr, xs, xsum, r.j, lane);
      // Each tile's 16 x 16 partial, one float4 per lane, in the tile's own
      // slot (row-group seg + q: J slots further on).
      const int J = S.J(r.g);
      float4_t xs4[4];
      if constexpr (FMT == QD_FMT_INT4_G64) group_sums(xr, xs4);
#pragma unroll
      for (int q = 0; q < U; ++q)
        if (q < r.nv) reinterpret_cast<float4_t*>(red)[(r.rel + q * J) * 64 + lane] = tile_mfma(t.w[q], xr, xs4);
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
      QD_PIN_ISSUE();
    }
    // The ring is consumed and refilled in slot order with a single loop
    // exit, so each compute waits only for its own slot's loads.
    for (;;) {
#pragma unroll
      for (int s = 0; s < D; ++s) {
        if (ref[s].g < ng) compute(s);
        ring[s] = next_tile(ref[s], lane);
          QD_PIN_ISSUE();
      }
      if (ref[0].g >= ng) break;   // slot 0 was refilled first: nothing left for later slots
    }
  } else {
    const int r = uni((int)(threadIdx.x >> 6)) - (kCtl - R);   // rank among reserve waves
    // The activations after group t are staged (one token row under glue:
    // their data has landed and the prologue pass, which every wave shares,
    // is starting).
    auto next_staged = [&](int t) {
      if constexpr (GLUE && MT == 1)
        if (lds_get(reinterpret_cast<const int*>(xsum) + 1) > t + 1) return true;
      return lds_get(staged) > t;
    };
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
        const uint32_t due = t0 + pace_ticks<FMT>((s * R + r) * (MT == 1 ? ku1(FMT) : U));
        while (!stop && (int32_t)((uint32_t)__builtin_amdgcn_s_memrealtime() - due) < 0) {
          stop = next_staged(trig);
          if (!stop) __builtin_amdgcn_s_sleep(2);
        }
        stop = stop || next_staged(trig);
        ring[s] = next_tile(ref[s], lane, !stop);
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

// Stage a group's multiplied vector in LDS.  All loads, and under a prologue
// the second operand's (gamma, or the gated product's B block) into
// xs + x_span(Kp), are issued before the single wait, so staging costs one
// memory round trip whatever K is.  The prologue then
// runs in place: each lane rewrites the 8-value chunks its own loads brought.
// POLICY: device-coherent for activations an earlier group of the step may
// have written (unless no cache can hold a stale copy of their lines); cached
// for the others, so the workgroups of an XCD share one L2 copy (8B step
// 1367-1372 vs 1375-1378 us coherent).
// One token row under a prologue, the element-wise pass (the gated product,
// or RMSNorm's normalisation once its factor r is known) is shared by all 16
// waves of the workgroup: chunk c (16 bytes) goes to wave (c / 64) % 16, and
// so is RMSNorm's sum of squares.  Every wave does its share before the
// group's barrier, so the pass is complete when the barrier releases the
// products.  The control wave stages the data, then publishes the group in
// pf[1] (pf: the LDS words after x); the compute waves wait for that in
// settle_to.
__device__ void prologue_share(const Sched& S, int g, int wave, int lane, half_t* xs, float* pf, int nrms) {
  const int Kp = S.J(g) * kSuperK;
  const int n4 = Kp / 8;                          // 16-byte chunks of x
  u32x4* x4 = reinterpret_cast<u32x4*>(xs);
  const u32x4* y4 = reinterpret_cast<const u32x4*>(xs + x_span(Kp));
  if (S.pro(g) == QD_PRO_GLU) {
    for (int c = 64 * wave + lane; c < n4; c += 64 * kWaves) x4[c] = glu8(x4[c], y4[c]);
    return;
  }
  // RMSNorm: each wave's sum of squares over its chunks (pf[4 + wave]), then,
  // once all 16 are in (pf[2] counts them, 16 per RMSNorm group so far),
  // their total in wave order.  The slots are reused by the next RMSNorm
  // group only after this group's barrier, which every wave reaches after
  // reading them.
  float ss = 0.0f;
  for (int c = 64 * wave + lane; c < n4; c += 64 * kWaves) ss = sumsq8(x4[c], ss);
  ss = wave_sum(ss);
  if (lane == 0) pf[4 + wave] = ss;
  __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
  int* const count = reinterpret_cast<int*>(pf) + 2;
  if (lane == 0) __hip_atomic_fetch_add(count, 1, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_WORKGROUP);
  for (uint32_t spins = 0; lds_get(count) < kWaves * nrms; ++spins) {
    if (spins > S.spin) {
      if (lane == 0) atomicOr(S.err, 2u);
      break;
    }
    __builtin_amdgcn_s_sleep(1);
  }
  __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
  float tot = 0.0f;
#pragma unroll
  for (int w = 0; w < kWaves; ++w) tot += pf[4 + w];
  const float r = rms_inverse(tot, S.k(g), S.eps(g));
  for (int c = 64 * wave + lane; c < n4; c += 64 * kWaves) x4[c] = rms8(x4[c], r, y4[c]);
}

template <bool GLUE, int POLICY = kPolicyCoherent>
__device__ __forceinline__ void stage_group_x(const Sched& S, int g, int lane, half_t* xs, float* pf, int& nrms) {
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
    if (pro != QD_PRO_NONE) {
      // The data before the flag; the compute waves read it after.
      __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
      if (lane == 0) lds_put(reinterpret_cast<int*>(pf) + 1, g + 1);
      if (pro == QD_PRO_RMSNORM) ++nrms;
      prologue_share(S, g, kCtl, lane, xs, pf, nrms);
    }
  } else {
    wait_stores();                                 // vmcnt(0): the data is in LDS
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
// of weight row rho (the MFMA output layout).  With GLUE: the member's
// epilogue applies, and in a paired group row-group rg is row-group rg / 2 of
// member rg % 2 (whose own copy is not written: the group writes the gated
// product instead).  h gets the stored values (0 for rows past the member and
// tokens past m); mi and n the member and the lane's row within it.
template <int FMT, bool GLUE>
__device__ __forceinline__ void store_rows16(const PlanArgs& p, const Sched& S, int g, int rg, int lane,
                                             float4_t v, bool paired, uint16_t (&h)[4], int& mi,
                                             int64_t& n) {
  mi = S.mem0(g);
  int64_t local;
  if (GLUE && paired) {
    mi += rg & 1;
    local = rg >> 1;
  } else {
    const int last = mi + S.nmem(g) - 1;
    while (mi < last && rg >= S.rg_begin(mi + 1)) ++mi;
    local = rg - S.rg_begin(mi);
  }
  const int gq = lane >> 4, rho = lane & 15;
  n = local * kTileRows + rho;
#pragma unroll
  for (int i = 0; i < 4; ++i) h[i] = 0;
  if (n >= S.n(mi)) return;
  uint16_t* const y = S.y(mi);
  uint16_t* const yt = GLUE && paired ? nullptr : S.yt(mi);
  const int epi = GLUE ? S.epi(mi) : (int)QD_EPI_NONE;
  const int64_t ld = S.ld(mi);
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = 4 * gq + i;
    if (tok < p.m) {
      const uint16_t hv = GLUE ? epilogue_bits(v[i], epi) : __builtin_bit_cast(uint16_t, (half_t)v[i]);
      h[i] = hv;
      __hip_atomic_store((__attribute__((address_space(1))) uint16_t*)(y + tok * ld + n), hv,
                         __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
      // The later group reading these outputs as its x finds them here in
      // matrix-core order too.
      if (yt)
        __hip_atomic_store((__attribute__((address_space(1))) uint16_t*)(yt + xt_index<FMT>(n, tok)),
                           hv, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// A paired group, rows n of its two members stored (a: the first member's
// values, b: the second's): the gated product fp16(a * b), one correctly
// rounded fp16 multiply, into the copy the consuming group reads, in
// matrix-core order.
template <int FMT>
__device__ __forceinline__ void store_product16(const PlanArgs& p, const Sched& S, int g, int lane, int64_t n,
                                                const uint16_t (&a)[4], const uint16_t (&b)[4]) {
  const int m0 = S.mem0(g);
  if (n >= S.n(m0)) return;
  uint16_t* const pt = S.yt(m0);
  const int gq = lane >> 4;
#pragma unroll
  for (int i = 0; i < 4; ++i) {
    const int tok = 4 * gq + i;
    if (tok < p.m) {
      const half_t u = __builtin_bit_cast(half_t, a[i]) * __builtin_bit_cast(half_t, b[i]);
      __hip_atomic_store((__attribute__((address_space(1))) uint16_t*)(pt + xt_index<FMT>(n, tok)),
                         __builtin_bit_cast(uint16_t, u), __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
  }
}

// This workgroup's sum-of-squares record of a member's outputs (see
// finish_group): sq holds, per lane (gq, rho), the squares of tokens
// 4 gq + i summed over the rows rho it stored, in row-group order; the 16
// lanes of a quarter are added in a fixed butterfly order and one lane per
// quarter writes its 4 tokens.
__device__ __forceinline__ void write_record(const PlanArgs& p, int rec, int lane, float4_t sq) {
#pragma unroll
  for (int s = 1; s < 16; s <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) sq[i] += __shfl_xor(sq[i], s);
  if ((lane & 15) == 0) {
    float* const dst = p.ss + (int64_t)rec * 16 + 4 * (lane >> 4);
#pragma unroll
    for (int i = 0; i < 4; ++i)
      __hip_atomic_store((__attribute__((address_space(1))) float*)(dst + i), sq[i], __ATOMIC_RELAXED,
                         __HIP_MEMORY_SCOPE_AGENT);
  }
}

// Spin (bounded) until the compute waves have counted `want` tiles against
// row-group slot `seg`.  After one timed-out wait (an error) later waits are
// skipped.
// The dynamic last group: claim chunks until this workgroup holds `want`
// (control wave only, one device-scope atomic per chunk, in order).  A claim
// past the last chunk, or the per-workgroup cap, ends the workgroup's part.
__device__ void dyn_take(const PlanArgs& p, DynCtl* d, uint32_t first, int n, int lane);

// The dynamic last group: claim chunks until this workgroup holds `want` (or
// the group is used up), all of them with one device-scope atomic: they are
// consecutive chunks (control wave only).
__device__ void dyn_claim(const PlanArgs& p, DynCtl* d, int want, int lane) {
  if (p.dyn_c <= 0 || lds_get(&d->ended)) return;
  const int n = min(want, p.dyn_max) - lds_get(&d->claimed);
  if (n <= 0) return;
  uint32_t first = 0;
  if (lane == 0)
    first = __hip_atomic_fetch_add(p.dyn_ctr + (p.epoch & 1), (uint32_t)n, __ATOMIC_RELAXED,
                                   __HIP_MEMORY_SCOPE_AGENT);
  dyn_take(p, d, (uint32_t)uni((int)first), n, lane);
}

// Record chunks first, first + 1, ... (n of them, claimed with one atomic) as
// this workgroup's next; those past the group end its part.
__device__ void dyn_take(const PlanArgs& p, DynCtl* d, uint32_t first, int n, int lane) {
  int have = lds_get(&d->claimed);
  bool used_up = false;
  for (int i = 0; i < n; ++i) {
    if (first + (uint32_t)i >= (uint32_t)p.dyn_nch || have >= p.dyn_max) {
      used_up = true;
      break;
    }
    if (lane == 0) d->chunk[have] = (int32_t)(first + (uint32_t)i);
    ++have;
  }
  if (lane == 0) {
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    lds_put(&d->claimed, have);
    if (used_up || have >= p.dyn_max) lds_put(&d->ended, 1);
  }
}

// Keep the claims dyn_q chunks ahead of the compute waves' hand-outs in the
// dynamic group (`handed`: the workgroup's tile counter).  Called from the
// control wave's waits, so a compute wave never waits on a claim for long.
template <int FMT>
__device__ __forceinline__ void dyn_service(const PlanArgs& p, const Sched& S, const uint32_t* handed,
                                            int lane) {
  if (p.dyn_c <= 0) return;
  const int last = p.ngroups - 1;
  const int h = (int)lds_get(handed) - S.off(last);   // hand-outs taken in the group
  if (h <= 0) return;
  const int per = p.dyn_c * ((S.J(last) + ku1(FMT) - 1) / ku1(FMT));
  const int want = (h - 1) / per + 1 + p.dyn_q;
  if (want > lds_get(&S.dyn->claimed)) dyn_claim(p, S.dyn, want, lane);
}

// Before the control wave waits at a barrier: the compute waves may take up
// to 64 more hand-outs before they all arrive (their rings and the reserve
// waves' hold fewer), and none may then wait on a claim; claim what those
// would need in the dynamic group.
template <int FMT>
__device__ __forceinline__ void dyn_ahead(const PlanArgs& p, const Sched& S, const uint32_t* handed, int lane) {
  if (p.dyn_c <= 0) return;
  const int last = p.ngroups - 1;
  const int h = (int)lds_get(handed) + 64 - S.off(last);
  if (h <= 0) return;
  const int per = p.dyn_c * ((S.J(last) + ku1(FMT) - 1) / ku1(FMT));
  dyn_claim(p, S.dyn, (h - 1) / per + 1 + p.dyn_q, lane);
}

template <int FMT>
__device__ __forceinline__ void wait_count(const PlanArgs& p, const Sched& S, const uint32_t* handed,
                                           const uint32_t* cnt, int seg, uint32_t want, bool& dead,
                                           int lane) {
  for (uint32_t spins = 0; !dead && lds_get(cnt + seg) < want; ++spins) {
    if (spins > p.spin_limit) {
      atomicOr(p.err, 2u);
      dead = true;
    }
    dyn_service<FMT>(p, S, handed, lane);
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
//
// Up to 16 token rows with glue, two more duties.  A member whose outputs a
// later RMSNorm reads has sum-of-squares records: this workgroup adds the
// squares of the values it stored, per token, and writes them as record
// ss + w (zeros if it stored none of them), before its stamp.  A paired group
// (row-groups alternate between its two members) writes the gated product of
// the two members' rows as each pair of row-groups completes.
//
// One token row, defer_last: the last row-group's rows are left in held /
// held_rg (-1: none) for the caller to store, rather than stored here.
template <int FMT, bool GLUE, int MT>
__device__ void finish_group(const PlanArgs& p, const Sched& S, int g, int w, int lane, const float* red,
                             uint32_t* cnt, int* stalled, bool& dead, const uint32_t* handed,
                             bool defer_last, float& held, int& held_rg) {
  int rec_mem = -1;                 // the member with sum-of-squares records, if any
  if constexpr (GLUE && MT != 1) {
    const int m0 = S.mem0(g), m1 = m0 + S.nmem(g);
    for (int mi = m0; mi < m1; ++mi)
      if (S.ss(mi) >= 0) rec_mem = mi;
  }
  float4_t sq = {0.0f, 0.0f, 0.0f, 0.0f};
  const int ntiles = S.tiles(g);
  if (ntiles == 0) {
    if (lane == 0) lds_put(stalled, g);
    if (GLUE && MT != 1 && rec_mem >= 0) write_record(p, S.ss(rec_mem) + w, lane, sq);
    return;
  }
  // Partials per row-group: one per tile at several token rows, one per
  // hand-out of ku1 tiles at one.
  const int J = MT == 1 ? (S.J(g) + ku1(FMT) - 1) / ku1(FMT) : S.J(g);
  const int rg0 = S.rg0(g), nseg = S.nseg(g);
  const int row = lane & 15, q = lane >> 4;
  const bool paired = GLUE && MT != 1 && S.paired(g);
  uint16_t first[4] = {0, 0, 0, 0};  // paired: the first member's stored values of the current pair
  for (int s = 0; s < nseg; ++s) {
    wait_count<FMT>(p, S, handed, cnt, s, (uint32_t)J, dead, lane);
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
      uint16_t h[4];
      int mi;
      int64_t n;
      store_rows16<FMT, GLUE>(p, S, g, rg0 + s, lane, sum, paired, h, mi, n);
      if constexpr (GLUE) {
        if (mi == rec_mem) {
#pragma unroll
          for (int i = 0; i < 4; ++i) {
            const float f = (float)__builtin_bit_cast(half_t, h[i]);
            sq[i] = __builtin_fmaf(f, f, sq[i]);
          }
        }
        if (paired) {
          // Workgroup ranges of a paired group start at even row-groups.
          if ((s & 1) == 0) {
#pragma unroll
            for (int i = 0; i < 4; ++i) first[i] = h[i];
          } else {
            store_product16<FMT>(p, S, g, lane, n, first, h);
          }
        }
      }
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
    if (defer_last && s == nseg - 1) {
      held = sum;
      held_rg = rg0 + s;
    } else if (lane < 16) {
      store_row<GLUE>(S, g, rg0 + s, row, sum);
    }
  }
  if (GLUE && MT != 1 && rec_mem >= 0) write_record(p, S.ss(rec_mem) + w, lane, sq);
}

// The dynamic last group (one token row): this workgroup's row-groups are
// those of the chunks it claimed, in claim order (local row-group s is
// row-group s mod C of chunk s / C).  Each is reduced, as in finish_group,
// once its hand-outs are counted; partial slots and counts are reused modulo
// their capacities (the compute waves wait before running that far ahead).
// Claims for the next chunks are made here, ahead of the hand-outs, until one
// finds the group used up.
template <int FMT, bool GLUE>
__device__ void finish_dynamic(const PlanArgs& p, const Sched& S, int g, int lane, const float* red,
                               uint32_t* cnt, int* stalled, bool& dead, const uint32_t* handed) {
  const int Ju = (S.J(g) + ku1(FMT) - 1) / ku1(FMT);
  const int C = p.dyn_c, R = S.R(g);
  const int rmask = p.dyn_rcap - 1, smask = p.dyn_scap - 1;
  const int row = lane & 15, q = lane >> 4;
  DynCtl* d = S.dyn;
  for (int s = 0; !dead; ++s) {
    const int k = s / C;
    dyn_claim(p, d, k + 1, lane);                     // chunk k, if there is one
    if (k >= lds_get(&d->claimed)) break;
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "workgroup", "local");
    const int ch = uni(d->chunk[k]);
    wait_count<FMT>(p, S, handed, cnt, s & smask, (uint32_t)Ju, dead, lane);
    float part = 0.0f;
    for (int t = q; t < Ju; t += 4) part += red[((s * Ju + t) & rmask) * 16 + row];
    const float sum = quad_reduce(part);
    if (lane == 0) cnt[s & smask] = 0u;
    const int rg = ch * C + (s - k * C);
    if (lane < 16 && rg < R) store_row<GLUE>(S, g, rg, row, sum);
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "workgroup", "local");
    if (lane == 0) lds_put(&d->reduced, s + 1);
  }
  if (lane == 0) lds_put(stalled, g);
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
// 2023, the chained step 2065 with 6 and 2085 with 8).  Re-measured once
// independent groups stopped waiting (only steps with dependent groups wait),
// wall us per step: one token row, 1 / 2 / 3 / 4 sleeps: chained 8B 1498 /
// 1489 / 1491 / 1497, glued 1670 / 1658 / 1654 / 1656; 16 token rows, 4 / 6
// / 8: chained 2029 / 2044 / 2075, glued 2214 / 2213 / 2223; on another
// device, 4 / 6: chained 2045 / 2056, glued 2207 / 2197 (6 kept: the two
// steps move in opposite directions by less than the spread between devices).
// One token row again with 9 reserve waves on rings of 2 and the glue passes
// shared, 1 / 2 / 3 / 4 sleeps: chained 1458-1460 / 1430-1433 / 1428-1430 /
// 1431-1436, glued 1576-1577 / 1548-1550 / 1538-1540 / 1541: 3 taken.
#ifndef QD_POLL_DELAY
#define QD_POLL_DELAY 3
#endif
#ifndef QD_POLL_DELAY16
#define QD_POLL_DELAY16 6
#endif
template <int FMT>
__device__ void wait_group(const PlanArgs& p, const Sched& S, const uint32_t* handed, int g, int lane,
                           int delay) {
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
    if (!done && kPollDepth == 1) dyn_service<FMT>(p, S, handed, lane);
  }
  wait_stores();                  // no poll left in flight
  asm volatile("" ::: "memory");
}

// Up to 16 token rows, a group under RMSNorm: stage gamma into LDS at xs and
// the 16 per-token factors r = 1 / sqrt(mean + eps) at rinv (0 past m).  Each
// token's sum of squares over x is the sum of the group's ss_n records (one
// per producing workgroup and row range, or one made before the step), added
// in a fixed order: lane l takes float4 l % 4 (tokens 4 (l % 4) .. + 3) of
// records l / 4, l / 4 + 16, ... in turn, then the lanes of equal l % 4 are
// added in a butterfly.  Gamma and the records are loaded first, with one
// wait.  Records are always read device-coherently (other workgroups wrote
// them in this launch); gamma as POLICY says.
template <int POLICY>
__device__ __forceinline__ void stage_rms16(const PlanArgs& p, const Sched& S, int g, int lane, half_t* xs,
                                            float* rinv) {
  const int Kp = S.J(g) * kSuperK;
  const int64_t k = S.k(g);
  dma_to_lds<POLICY>(make_rsrc(S.gamma(g), (uint32_t)(k * 2)), Kp, lane, xs);
  const int nrec = S.ss_n(g);
  const __amdgpu_buffer_rsrc_t rr = make_rsrc(p.ss + (int64_t)S.ss0(g) * 16, (uint32_t)nrec * 64u);
  const int tq = lane & 3, r0 = lane >> 2;
  float4_t acc = {0.0f, 0.0f, 0.0f, 0.0f};
  for (int i0 = 0; i0 < nrec; i0 += 128) {
    u32x4 v[8];
#pragma unroll
    for (int u = 0; u < 8; ++u) v[u] = bload16_coherent(rr, (uint32_t)((i0 + 16 * u + r0) * 64 + tq * 16));
#pragma unroll
    for (int u = 0; u < 8; ++u) {
      const float4_t f = __builtin_bit_cast(float4_t, v[u]);
#pragma unroll
      for (int i = 0; i < 4; ++i) acc[i] += f[i];
    }
  }
#pragma unroll
  for (int s = 4; s < 64; s <<= 1)
#pragma unroll
    for (int i = 0; i < 4; ++i) acc[i] += __shfl_xor(acc[i], s);
  wait_stores();                  // vmcnt(0): gamma is in LDS
  if (lane < 4) {
#pragma unroll
    for (int i = 0; i < 4; ++i) {
      const int tok = 4 * lane + i;
      rinv[tok] = tok < p.m ? rms_inverse(acc[i], k, S.eps(g)) : 0.0f;
    }
  }
}

template <int FMT, bool GLUE, int MT>
__device__ void control_wave(const PlanArgs& p, const Sched& S, int w, int lane, half_t* xs,
                             float* xsum, const float* red, uint32_t* cnt, int* stalled,
                             int* staged, const uint32_t* handed) {
  // The control wave is on every group's critical path: let it issue ahead of
  // the compute waves that share its SIMD.
  __builtin_amdgcn_s_setprio(3);
  int nrms = 0;                   // RMSNorm prologues staged (one token row, glue)
  // The dynamic last group's chunks are claimed ahead of the hand-outs: in
  // the control wave's waits, and before each of its barriers for what the
  // compute waves could take while it waits there (dyn_ahead), so that no
  // compute wave waits on a claim while the control wave waits at a barrier.
  // Group 0's activations: nothing of this launch has written anything yet
  // (earlier launches' writes are visible at kernel start).
  if constexpr (MT == 1) stage_group_x<GLUE, kPolicyDefault>(S, 0, lane, xs, xsum, nrms);
  if constexpr (MT == 1) dyn_ahead<FMT>(p, S, handed, lane);
  if constexpr (MT != 1 && GLUE)
    if (S.pro(0) == QD_PRO_RMSNORM) stage_rms16<kPolicyDefault>(p, S, 0, lane, xs, xsum);
  wg_barrier();                   // activations of group 0 staged
  bool dead = false;
  for (int g = 0; g < p.ngroups; ++g) {
    // The boundary before an independent group g + 1 does not wait.  With a
    // lag L, this workgroup instead waits, while it streams g, for every
    // workgroup to have finished group g - L, so none runs more than about L
    // groups ahead of the slowest.  (Measured: on the larger steps, workgroups
    // left to drift apart end the step later than with a wait at every
    // boundary; on the smaller ones they end it earliest.)
    if (p.lag > 0 && g + 1 < p.ngroups && (S.order(g + 1) & kIndependent) && g >= p.lag)
      wait_group<FMT>(p, S, handed, g - p.lag, lane, 0);
    bool dynamic = false;
    if constexpr (MT == 1) {
      if (p.dyn_c > 0 && g == p.ngroups - 1) {
        finish_dynamic<FMT, GLUE>(p, S, g, lane, red, cnt, stalled, dead, handed);
        dynamic = true;
      }
    }
    // One token row, a step with a dynamic last group, 6 GiB of weights or
    // more and no drift bound (so below 12 GiB; p.defer), before a group whose activations no earlier
    // group writes and that waits for no other workgroup, g's outputs needing
    // no acknowledgement: the last row-group's rows are stored after the next
    // activations are staged, so the staging's wait (vmcnt(0)) covers its own
    // loads and not those stores.  Measured, wall us per step, stores before /
    // after the staging, on three devices: 8B int8 1202 / 1192, 1221 / 1195,
    // 1203 / 1190.  Elsewhere it was slower: 27B-shaped int8 (drift bound 3)
    // 3672 / 3700, 8B INT4 759 / 804, 4B int8 735 / 761, 2B int8 344 / 375
    // (and, with the staging issued before the last row-group's reduction
    // instead, 8B int8 1205 / 1202, INT4 760 / 850, 4B 733 / 770, 2B 344 /
    // 381).
    const bool defer = MT == 1 && p.defer && p.lag == 0 && g + 1 < p.ngroups &&
                       !(S.order(g) & kAckOutputs) &&
                       (S.order(g + 1) & (kStageEarly | kNoWait)) == (kStageEarly | kNoWait);
    float held = 0.0f;
    int held_rg = -1;
    if (!dynamic)
      finish_group<FMT, GLUE, MT>(p, S, g, w, lane, red, cnt, stalled, dead, handed, defer, held, held_rg);
    publish(p, S, g, w, lane);
    if (g + 1 < p.ngroups) {
      // Activations no earlier group writes are staged while the stamps are
      // awaited; the others only once every workgroup has finished g.  The
      // compute waves start g + 1 after the barrier either way.
      // (MT > 1: the compute waves read the activations themselves.)
      const bool early = (S.order(g + 1) & kStageEarly) != 0;
      // Several token rows under RMSNorm: gamma and the per-token factors,
      // whose records are complete once every workgroup has finished the
      // producing group (or were made before the step: early).
      const bool rms16 = GLUE && MT != 1 && S.pro(g + 1) == QD_PRO_RMSNORM;
      if (MT == 1 && early) stage_group_x<GLUE, kPolicyDefault>(S, g + 1, lane, xs, xsum, nrms);
      if (defer && held_rg >= 0 && lane < 16) store_row<GLUE>(S, g, held_rg, lane, held);
      if (rms16 && early) stage_rms16<kPolicyDefault>(p, S, g + 1, lane, xs, xsum);
      // A further row range of the same op(s) reads nothing group g writes,
      // and needs what g needed, which g's own boundary already waited for;
      // a group independent of every earlier group needs nothing of them.
      if (!(S.order(g + 1) & kNoWait))
        wait_group<FMT>(p, S, handed, g, lane, MT > 1 ? QD_POLL_DELAY16 : early ? 0 : QD_POLL_DELAY);
      if (MT == 1 && !early) {
        if (S.order(g + 1) & kCleanLines) stage_group_x<GLUE, kPolicyDefault>(S, g + 1, lane, xs, xsum, nrms);
        else stage_group_x<GLUE>(S, g + 1, lane, xs, xsum, nrms);
      }
      if (rms16 && !early) {
        if (S.order(g + 1) & kCleanLines) stage_rms16<kPolicyDefault>(p, S, g + 1, lane, xs, xsum);
        else stage_rms16<kPolicyCoherent>(p, S, g + 1, lane, xs, xsum);
      }
      if (lane == 0) lds_put(staged, g + 1);
      if constexpr (MT == 1) dyn_ahead<FMT>(p, S, handed, lane);
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
  // The dynamic last group's claims follow the counter and the flags.
  S.dyn = reinterpret_cast<DynCtl*>(next + 4);
  S.dyn_c = p.dyn_c;
  S.dyn_rmask = p.dyn_rcap - 1;
  S.dyn_smask = p.dyn_scap - 1;
  S.dyn_win = p.dyn_win;
  S.spin = p.spin_limit;
  S.err = p.err;
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
      if (MT == 1 && GLUE) {
        reinterpret_cast<int*>(xsum)[1] = 0;      // no prologue staged yet
        reinterpret_cast<int*>(xsum)[2] = 0;      // no RMSNorm shares counted
      }
      S.dyn->claimed = 0;
      S.dyn->ended = 0;
      S.dyn->reduced = 0;
      // The next run's claim counter (this run uses the other one).
      if (p.dyn_c > 0 && w == 0)
        __hip_atomic_store(p.dyn_ctr + ((p.epoch + 1) & 1), 0u, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    }
    for (int i = threadIdx.x; i < p.cnt_bytes / 4; i += kWaves * 64) cnt[i] = 0u;
  }
  __syncthreads();

  if (wave == kCtl) {
    control_wave<FMT, GLUE, MT>(p, S, w, lane, xs, xsum, red, cnt, stalled, staged, next);
  } else {
    const int last = p.ngroups - 1;
    // The dynamic last group has no set length: its hand-outs end where the
    // claims do.
    const int total = p.dyn_c > 0 ? 0x3fffffff : S.off(last) + S.tiles(last);
    if (wave < kCtl - R)
      compute_wave<FMT, D, false, R, MT, U, GLUE>(p, S, total, next, lane, xs, xsum, red, cnt, stalled, staged);
    else
      compute_wave<FMT, RS, true, R, MT, U, GLUE>(p, S, total, next, lane, xs, xsum, red, cnt, stalled, staged);
  }
  __builtin_amdgcn_s_waitcnt(0);
}

// Before a step with up to 16 token rows: copy the activations no group of
// the step writes into matrix-core order (see load_xblock), 256 chunks of 16
// bytes per workgroup, chunk-contiguous stores.  Chunks of token rows past m
// or past K are left as they are (zero since the plan was made).  Under a
// gated product the copy holds fp16(A * B) of the two blocks.  A job with a
// record instead (one workgroup) writes each token's sum of squares over its
// K values, for a group under RMSNorm: per token one wave adds its lanes'
// 8-value chunks in order, then the lanes in a butterfly.
struct XtJob {          // 48 bytes
  const uint16_t* x;    // [m, k]; under a gated product [2, m, k]
  uint16_t* t;          // the copy (copy jobs)
  float* ss;            // the record, 16 floats (record jobs), or null
  int64_t k;
  int64_t first_block;  // first workgroup of this job
  int32_t glu;          // copy jobs: 1 = the copy holds the gated product
  int32_t pad;
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
  if (jb.ss) {
    const int wave = threadIdx.x >> 6, lane = threadIdx.x & 63;
    for (int tok = wave; tok < 16; tok += 4) {
      float acc = 0.0f;
      if (tok < m)
        for (int64_t i = lane * 8; i < jb.k; i += 512)
          acc = sumsq8(*reinterpret_cast<const u32x4*>(jb.x + tok * jb.k + i), acc);
      acc = wave_sum(acc);
      if (lane == 0) jb.ss[tok] = acc;
    }
    return;
  }
  // chunk c = (8 j + q) 64 + lane, lane = 16 gq + t
  const int64_t c = ((int64_t)blockIdx.x - jb.first_block) * 256 + threadIdx.x;
  const int tok = (int)(c & 15), gq = (int)((c >> 4) & 3), q = (int)((c >> 6) & 7);
  if constexpr (FMT == QD_FMT_INT8_B32) {
    const int64_t k = (c >> 9) * kSuperK + kpos<FMT>(q, gq);
    if (tok >= m || k >= jb.k) return;
    u32x4 v = *reinterpret_cast<const u32x4*>(jb.x + tok * jb.k + k);
    if (jb.glu) v = glu8(v, *reinterpret_cast<const u32x4*>(jb.x + (m + tok) * jb.k + k));
    *reinterpret_cast<u32x4*>(jb.t + c * 8) = v;
  } else {
    // Both halves of the lane's 16 values (K is a multiple of 64, so the
    // second half is in range with the first), then the operand's pairs.
    const int64_t k = (c >> 9) * kSuperK + kpos<FMT>(q & ~1, gq);
    if (tok >= m || k >= jb.k) return;
    u32x4 h0 = *reinterpret_cast<const u32x4*>(jb.x + tok * jb.k + k);
    u32x4 h1 = *reinterpret_cast<const u32x4*>(jb.x + tok * jb.k + k + 8);
    if (jb.glu) {
      h0 = glu8(h0, *reinterpret_cast<const u32x4*>(jb.x + (m + tok) * jb.k + k));
      h1 = glu8(h1, *reinterpret_cast<const u32x4*>(jb.x + (m + tok) * jb.k + k + 8));
    }
    *reinterpret_cast<u32x4*>(jb.t + c * 8) = (q & 1) ? int4_hi(h0, h1) : int4_lo(h0, h1);
  }
}

// Streaming ring depth per format (tiles per streaming wave), measured.
// int8 steps with stalls: rings of 2 with 9 reserve waves (wall us per step,
// rings of 3 / 2 and reserve tiles 1 / 3 on rings of 3: chained 8B 1441 /
// 1429 / 1497 / 1463-1468, glued 1554 / 1546 / 1611-1615 / 1545).
#ifndef QD_PLAN_RING8
#define QD_PLAN_RING8 2
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
  bool glue = false;                     // a prologue or an epilogue in the persistent part
  bool light = false;                    // no group waits for the one before it: the lighter reserve (kernel_ptr)
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
  bool cooperative = false;              // launch cooperatively (after a run whose wait timed out)
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
  // Several token rows with glue:
  std::vector<int> rec;        // per member: key of its sum-of-squares records, or -1
  int ss_key = -1;             // under RMSNorm: key of the records of x
  bool ss_early = false;       // ... made before the step (x is not written by the step)
  bool paired = false;         // two members whose gated product a later group reads
  int64_t glu_src = -1;        // under the gated product: the paired group writing it, or -2 when
                               // x is not written by the step (the product is copied before it)
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
    // A group that reads nothing an earlier group writes, and writes nothing
    // an earlier group reads or writes, needs no earlier group to have
    // finished: the device-wide wait before it is skipped.  (A later group
    // that does depend on an earlier one waits for every workgroup to finish
    // the group before it, and a workgroup finishes its groups in order.)
    bool independent = early;
    for (size_t j = 0; independent && j < i; ++j) {
      const uint64_t xbj = (uint64_t)m * gs[j].k * 2 * (gs[j].pro == QD_PRO_GLU ? 2 : 1);
      for (const PMember& pa : gs[i].mem) {
        const uint64_t ya = y_span(pa, m);
        if (ranges_overlap(pa.y, ya, gs[j].x, xbj) ||
            (gs[j].pro == QD_PRO_RMSNORM && ranges_overlap(pa.y, ya, gs[j].gamma, (uint64_t)gs[j].k * 2)))
          independent = false;
        for (const PMember& pj : gs[j].mem)
          if (ranges_overlap(pa.y, ya, pj.y, y_span(pj, m))) independent = false;
      }
    }
    if (independent && i > 0) gs[i].order |= kNoWait | kIndependent;
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

// A paired group's row range per piece of the split below, in row-groups:
// whole pairs, at most tiles / J row-groups per workgroup, and, when the
// group has to be cut, a multiple of 32 row-groups (256 rows of each member),
// so that the gated product's copy is addressed by plain offsets.  0 if no
// such piece exists.
int64_t paired_piece(int64_t R, int J, int64_t tiles, int G) {
  const int64_t pairs = tiles / J / 2;
  if (pairs < 1) return 0;
  const int64_t full = pairs * 2 * G;
  return R <= full ? full : full / 32 * 32;
}

// Split groups into row ranges of at most `tiles` tiles per workgroup (G
// workgroups), so that one range's 16 x 16 tile partials fit in LDS.  Each
// range is a group of its own whose members are the slices of the original
// members it covers; ranges after the first carry kNoWait.  A paired group's
// ranges hold the same rows of both members.  False if a single row-group
// (a paired group: a pair) has more tiles than that.
bool split_rows(std::vector<HostGroup>& gs, int64_t tiles, int G, int64_t tbytes) {
  std::vector<HostGroup> out;
  for (HostGroup& hg : gs) {
    const int64_t per_wg = tiles / hg.J;
    if (per_wg < 1) return false;
    const int64_t piece = hg.paired ? paired_piece(hg.R, hg.J, tiles, G) : per_wg * G;
    if (piece < 1) return false;
    if (hg.R <= piece) {
      out.push_back(std::move(hg));
      continue;
    }
    for (int64_t a = 0; a < hg.R; a += piece) {
      const int64_t b = std::min<int64_t>(hg.R, a + piece);
      HostGroup pg = hg;
      pg.mem.clear();
      pg.src.clear();
      pg.yt_off.clear();
      pg.rec.clear();
      pg.R = 0;
      for (size_t q = 0; q < hg.mem.size(); ++q) {
        const PMember& mm = hg.mem[q];
        // Row-groups [lo, hi) of the group that are this member's, and how
        // many of the member's come before them.
        int64_t lo, hi, skip;
        if (hg.paired) {          // a and b are even; both members have R / 2 row-groups
          lo = a / 2;
          hi = b / 2;
          skip = lo;
        } else {
          const int64_t r0 = mm.rg_begin, r1 = r0 + ceil_div(mm.n, kTileRows);
          lo = std::max(a, r0);
          hi = std::min(b, r1);
          skip = lo - r0;
        }
        if (lo >= hi) continue;
        PMember slice = mm;
        slice.blob = mm.blob + skip * hg.J * tbytes;
        slice.y = mm.y + skip * kTileRows;
        slice.n = std::min<int64_t>(mm.n - skip * kTileRows, (hi - lo) * kTileRows);
        slice.rg_begin = pg.R;
        pg.mem.push_back(slice);
        pg.src.push_back(hg.src[q]);
        pg.yt_off.push_back(hg.yt_off[q] < 0 ? -1 : hg.yt_off[q] + skip * kTileRows * 16 * 2);
        pg.rec.push_back(hg.rec[q]);
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

// Reserve waves (and tiles each) per format, as measured on MI355X.  int8
// (the steps with stalls: some group waits for the one before it): 9 reserve
// waves of 2 tiles.  Re-measured with the current kernel on two devices,
// wall us per step, reserve waves 3 / 5 / 7 / 8 / 9 / 10 / 11: chained 8B
// 1578 / 1562 / 1470-1477 / 1469-1470 / 1433-1439 / 1553-1556 / 1719, glued
// 1690 / 1652-1657 / 1560-1568 / 1562 / 1552-1555 / 1684 / 1842.  Before,
// 7 of 2 tiles (8 streaming waves, two to a SIMD) was best for the 2B-, 4B-
// and 8B-shaped steps alike (15 to 50 tiles per workgroup per group).  More reserve tiles run several groups
// ahead and are then not free for the next stall; fewer leave memory idle
// for part of it.  INT4: rings of 2 tiles per streaming wave and 4 reserve
// waves of 2 tiles (measured with the one-AND decode and the plain launch,
// 8B INT4 step, us: reserve 0 914, 2 x 2 915, 3 x 2 902, 4 x 2 900, 5 x 2 924,
// 6 x 2 965, 3 x 3 924, 4 x 3 925; rings of 3 and 4 without reserve 965 and
// 1024).
#ifndef QD_PLAN_RESERVE4
#define QD_PLAN_RESERVE4 4
#endif
#ifndef QD_PLAN_RESERVE4_S
#define QD_PLAN_RESERVE4_S 1
#endif
constexpr int kReserveInt4 = QD_PLAN_RESERVE4, kReserveInt4S = QD_PLAN_RESERVE4_S;

#ifndef QD_PLAN_RESERVE8_R
#define QD_PLAN_RESERVE8_R 9
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
// Reserve waves at several token rows: 3 of one unit (int8) and 1 (INT4)
// since independent groups stopped waiting; measured (HIP-event medians, us,
// 7 / 3 / 0 reserve waves for int8, 3 / 1 / 0 for INT4): 8B int8 1863 / 1809
// / 1842, 8B INT4 1300 / 1273 / 1289, 27B-shaped int8 6303 / 6119 / 6280,
// glued 8B int8 2253 / 2188 / 2294.  (Before, with a wait at every boundary,
// 7 and 3 were best; see below.)
#ifndef QD_PLAN_RESERVE16_R
#define QD_PLAN_RESERVE16_R 3
#endif
// int8 at several token rows, a step in which some group waits for the one
// before it (more stalls to cover): 4 reserve waves.  Measured, wall us per
// step, 3 / 4 / 5 reserve waves: chained 8B 2070-2082 / 2034-2049 /
// 2031-2046, glued 8B 2211-2213 / 2194-2197 / 2213-2214 (on another device
// 3 / 4: chained 2080 / 2043-2048, glued 2227-2230 / 2228-2230); the steps without
// waits kept 3 (8B 1711-1717 / 1722-1724 / 1747-1752, 27B-shaped 5420-5423 /
// 5444 / 5473-5477; 2 reserve waves: 8B 1712-1720, chained 2122).
#ifndef QD_PLAN_RESERVE16_WAITS_R
#define QD_PLAN_RESERVE16_WAITS_R 4
#endif
#ifndef QD_PLAN_UNIT16
#define QD_PLAN_UNIT16 2
#endif
#ifndef QD_PLAN_RESERVE16_S
#define QD_PLAN_RESERVE16_S 1
#endif
// INT4 at up to 16 token rows: its own shape (tiles of 2304 rather than 4352
// bytes), measured on the 8B INT4 step with a wait at every boundary (us):
// reserve waves of one unit
// 0 / 2 / 3 / 4 / 5 / 6 / 7 / 10 gave 1671 / 1608 / 1607 / 1621-1634 / 1630 /
// 1650 / 1709 / 2038 (from two devices); units of 3 row-groups 1636 with 4
// reserve waves.  A ring of 2 units, two units per reserve wave and units of
// 4 spill registers.
#ifndef QD_PLAN_RING16_INT4
#define QD_PLAN_RING16_INT4 QD_PLAN_RING16
#endif
#ifndef QD_PLAN_RESERVE16_INT4_R
#define QD_PLAN_RESERVE16_INT4_R 1
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

// Glue: at one token row the staging applies the prologue in LDS; at several
// the compute waves apply RMSNorm to each activation block and a gated
// product is read from a copy that holds it.  The row stores apply the
// epilogue.  (Separate instances, so steps without glue run the plain
// kernels.)
template <int FMT, bool GLUE>
const void* multi_kernel(bool light) {
  if constexpr (FMT == QD_FMT_INT8_B32)
    return light ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, QD_PLAN_RING16, QD_PLAN_RESERVE16_R,
                                                               QD_PLAN_RESERVE16_S, GLUE, 16, QD_PLAN_UNIT16>)
                 : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, QD_PLAN_RING16,
                                                               QD_PLAN_RESERVE16_WAITS_R, QD_PLAN_RESERVE16_S,
                                                               GLUE, 16, QD_PLAN_UNIT16>);
  else
    return reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT4_G64, QD_PLAN_RING16_INT4, QD_PLAN_RESERVE16_INT4_R,
                                                       QD_PLAN_RESERVE16_INT4_S, GLUE, 16, QD_PLAN_UNIT16_INT4>);
}

//
// `light`: no group waits for the one before it (few stalls to cover).  At
// several token rows it picks the int8 reserve (above).  At one token row
// without glue: no reserve waves, every compute wave streaming (int8 with
// rings of 2 tiles).  Measured on those steps (HIP-event medians, us):
// first, reserve 7 x 2 / 3 x 2 / none for int8, 4 x 2 / none for INT4: 4B
// int8 781 / 741 / 770, 27B-shaped int8 3954 / 3866 / 3879, 8B INT4 813 /
// 772; with the rotated ranges, 8B int8 without a drift bound 1283 / 1246
// (7 x 2 / 3 x 2).  Then, with the matrix-core tiles and the dynamic head,
// int8 reserve 3 x 2 on rings of 3 / none on rings of 3 / none on rings of 2:
// 8B 1266 / 1220 / 1216, 2B 365 / 349 / 341, 4B 727 / 740 / 728, 27B-shaped
// 3651-3663 / 3661-3664 / 3653 (and 2 x 2 reserve 1239, 4 x 2 1285 on the 8B
// step).  Steps with stalls keep the deeper reserve and rings of 3 (the
// chained 8B step, reserve 7 / 5 / 3 / 0 waves of 2: 1485 / 1575 / 1596 /
// 1644; the glued one 1640 / 1718 / 1741 / 1791).  Later, with the stores
// after the staging: int8 rings of 1 / 2 / 3 without reserve (2 x 2 reserve
// on rings of 2): 2B 342-343 / 349-350 / 357 (355), 4B 721-722 / 730-731 /
// 749-750 (718), 8B 1215-1217 / 1192-1193 / 1192-1193 (1206-1207); so steps
// with a dynamic last group and 6 GiB of weights or more (`big`, the plan's
// defer) keep rings of 2 and the others take rings of 1.
#ifndef QD_PLAN_RESERVE8_LIGHT
#define QD_PLAN_RESERVE8_LIGHT 0
#endif
#ifndef QD_PLAN_RING8_LIGHT
#define QD_PLAN_RING8_LIGHT 2
#endif
#ifndef QD_PLAN_RING8_LIGHT_SMALL
#define QD_PLAN_RING8_LIGHT_SMALL 1
#endif
#ifndef QD_PLAN_RESERVE4_LIGHT
#define QD_PLAN_RESERVE4_LIGHT 0
#endif
const void* kernel_ptr(int fmt, bool multi, bool glue, bool light, bool big) {
  if (multi) {
    if (fmt == QD_FMT_INT8_B32)
      return glue ? multi_kernel<QD_FMT_INT8_B32, true>(light) : multi_kernel<QD_FMT_INT8_B32, false>(light);
    return glue ? multi_kernel<QD_FMT_INT4_G64, true>(light) : multi_kernel<QD_FMT_INT4_G64, false>(light);
  }
  if (light && !glue) {
    if (fmt == QD_FMT_INT8_B32)
      return big ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, QD_PLAN_RING8_LIGHT,
                                                               QD_PLAN_RESERVE8_LIGHT, kReserve8S, false, 1, 1>)
                 : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, QD_PLAN_RING8_LIGHT_SMALL,
                                                               QD_PLAN_RESERVE8_LIGHT, kReserve8S, false, 1, 1>);
    return reinterpret_cast<const void*>(
        &stack_kernel<QD_FMT_INT4_G64, kRing4, QD_PLAN_RESERVE4_LIGHT, kReserveInt4S, false, 1, 1>);
  }
  if (fmt == QD_FMT_INT8_B32)
    return glue ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, kRing8, kReserve8R, kReserve8S, true, 1, 1>)
                : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT8_B32, kRing8, kReserve8R, kReserve8S, false, 1, 1>);
  return glue ? reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT4_G64, kRing4, kReserveInt4, kReserveInt4S, true, 1, 1>)
              : reinterpret_cast<const void*>(&stack_kernel<QD_FMT_INT4_G64, kRing4, kReserveInt4, kReserveInt4S, false, 1, 1>);
}

// A job made before each step at several token rows: a copy of an activation
// no group of the step writes, in matrix-core order (of x, or of the gated
// product of its two blocks), or the sum-of-squares record of such an
// activation under RMSNorm.
struct HostJob {
  const uint16_t* x;
  int64_t k;
  int64_t copy_off;            // byte offset of the copy in the plan's copies, or -1 (a record job)
  int64_t rec;                 // the record (record jobs), or -1
  int32_t glu;                 // copy jobs: the copy holds the gated product of x's two blocks
  int64_t first_block;
};

// The persistent step's tables, built on the host alone: the groups in step
// order with their boundary ordering, their row-range split at several token
// rows, the activation-copy slots, the sum-of-squares records, the
// per-workgroup schedules and the LDS the kernel needs, for G workgroups.
// Copy addresses are byte offsets into the plan's copies until those exist.
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
  std::vector<HostJob> jobs;   // made before each step
  int64_t xt_total = 0, xt_blocks = 0;
  int64_t ss_total = 0;        // sum-of-squares records, 16 floats each
  size_t x_bytes = 0, xsum_bytes = 0, red_bytes = 0, cnt_bytes = 0, tab_bytes = 0, lds = 0;
  int lag = 0;                 // drift bound across independent groups, in groups (0: none)
  bool light = false;          // see kernel_ptr
  // The dynamic last group (one token row; see PlanArgs), dyn_c = 0 if none.
  int dyn_c = 0, dyn_q = 0, dyn_nch = 0, dyn_max = 0, dyn_rcap = 0, dyn_scap = 0, dyn_win = 0;
  // A dynamic last group and 6 GiB of weights or more: stores after the
  // staging (control_wave) and rings of 2 for the light int8 step (kernel_ptr).
  bool defer = false;
};

int pow2_at_least(int64_t v) {
  int p = 1;
  while (p < v) p <<= 1;
  return p;
}

// The last group before g writing any byte of [x, x + xb), or SIZE_MAX.
size_t last_writer(const std::vector<HostGroup>& gs, size_t g, const void* x, uint64_t xb, int64_t m) {
  size_t p = SIZE_MAX;
  for (size_t j = 0; j < g; ++j)
    for (const PMember& pj : gs[j].mem)
      if (ranges_overlap(x, xb, pj.y, y_span(pj, m))) p = j;
  return p;
}

// How many groups the slowest workgroup may trail before a workgroup starting
// an independent group waits for it (0: no bound), by the step's weight bytes
// and token rows.  Measured on the persistent steps here (HIP-event medians,
// us; a wait at every boundary / none / lags of 1, 3 and 6 groups):
//   2B int8, 1.8 GB, one row:          561 /  451 /  520 /  535 /  516
//   4B int8, 3.9 GB, one row:          926 /  777 /  850 /  857 /  888
//   8B INT4, 4.3 GB, one row:          896 /  816 /  818 /  857 /  865
//   8B INT4, 4.3 GB, 16 rows:         1599 / 1299 / 1375 / 1396 / 1321
//   8B int8, 8.0 GB, one row:         1330 / 1348 / 1267 / 1298 / 1317
//   8B int8, 8.0 GB, 16 rows:         1997 / 1855 / 1979 / 1889 / 1856
//   27B-shaped int8, 24.5 GB, one row: 4250 / 4718 / 4011 / 3940 / 3989
//   27B-shaped int8, 24.5 GB, 16 rows: 6432 / 6516 / 6419 / 6225 / 6267
// Those one-row figures were taken before the one-row ranges of unevenly
// divided groups rotated (layout_plan), when the same workgroups carried the
// extra row-groups of every layer.  With the rotation (no bound / lags of 1,
// 2 and 3 groups; reserve as `light` chooses, except where marked):
//   2B int8, one row:            357 /  486 /  501 /  501
//   4B int8, one row:            725 /  892 /  859 /  867
//   8B INT4, one row:            758 /  957 /  927 /  885
//   8B int8, one row:           1246 / 1340 / 1322 / 1304  (7 x 2 reserve: no bound 1283,
//                                                          lag 1 1259, lag 2 1294)
//   27B-shaped int8, one row:   3767 / 3964 / 3757 / 3668
// With the stores after the staging, the fixed head for steps with waits and
// rings of 1 for the small steps (wall us per step; lags of 2 / 3 / 5 / 8 /
// 12 / 16 / 24 groups): 27B-shaped int8, one row, 3815 / 3668-3685 / 3686-
// 3707 / 3613-3623 / 3594-3599 / 3583-3591 / 3611-3654; at 16 rows lag 3 /
// 16: 5417-5422 / 5342.  The smaller steps still do best without a bound
// (no bound / lags of 16 / 32: 8B int8 1195 / 1232 / 1222, 8B INT4 746-748 /
// 835 / 821-824, 4B 741 / 841 / 824, 2B 343 / 460 / 442).
int drift_lag(int64_t weight_bytes, bool multi) {
  (void)multi;
  if (weight_bytes >= ((int64_t)12 << 30)) return 16;
  return 0;
}

// `scratch`: whether the plan has scratch of its own (a plan object).  Steps
// with several token rows then keep activation copies in matrix-core order,
// and take glue, which needs those copies and sum-of-squares records;
// without scratch every activation is read in place, and glue at several
// token rows ends the persistent part of the step.
void layout_plan(const qd_linear_op* ops, int64_t n_ops, int64_t m, int G, PlanLayout* L,
                 bool scratch = true) {
  *L = PlanLayout{};
  L->G = G;
  // Persistent walker: one format, no empty-K groups, up to 16 token rows.
  // The leading groups that qualify run in the persistent kernel; from the
  // first group that does not (another format, say an fp16 head, or glue at
  // several token rows the kernel cannot take), the rest of the step is
  // replayed as per-group launches after it on the same stream.
  std::vector<HostGroup> groups;
  const bool multi = m > 1;
  if (m < 1 || m > 16 || G < 1 || G > kMaxWorkgroups) return;
  int fmt = 0;
  int64_t split = n_ops;
  for (int64_t i = 0; i < n_ops;) {
    int64_t e = i + 1;
    while (e < n_ops && ops[e].group == ops[i].group) ++e;
    HostGroup hg{ops[i].x, ops[i].w.k, (int)ceil_div(ops[i].w.k, kSuperK), {}, {}, {}, 0,
                 ops[i].gamma, ops[i].prologue, ops[i].eps};
    bool gok = true;
    int gfmt = fmt;
    for (int64_t q = i; q < e; ++q) {
      if (ops[q].w.n == 0) continue;
      if (ops[q].w.k == 0) gok = false;
      if (gfmt == 0) gfmt = ops[q].w.fmt;
      if (ops[q].w.fmt != gfmt) gok = false;
      if (gfmt != QD_FMT_INT8_B32 && gfmt != QD_FMT_INT4_G64) gok = false;   // fp16: replay
      if (multi && !scratch && (ops[q].prologue != QD_PRO_NONE || ops[q].epilogue != QD_EPI_NONE)) gok = false;
      hg.mem.push_back(PMember{static_cast<const uint8_t*>(ops[q].w.data), ops[q].y, ops[q].w.n,
                               hg.R, ops[q].epilogue, (int32_t)ops[q].w.n, -1, nullptr});
      hg.src.push_back(i);
      hg.yt_off.push_back(-1);
      hg.rec.push_back(-1);
      hg.R += (int)ceil_div(ops[q].w.n, kTileRows);
    }
    if (!gok) {
      split = i;
      break;
    }
    fmt = gfmt;
    if (!hg.mem.empty()) groups.push_back(std::move(hg));
    i = e;
  }
  if (groups.empty()) return;
  order_groups(groups, m, tile_bytes(fmt));

  // Several token rows with glue: what each glued group needs.
  //  * RMSNorm needs each token's sum of squares over x.  When no group of
  //    the step writes x, it is summed before the step (one record); when x
  //    is exactly the whole output of one op of its last writer, that op's
  //    workgroups write one record each as they finish it.  The op must be
  //    the only one of its group with records, in a group that is not paired.
  //  * The gated product needs its two blocks as the whole outputs of the two
  //    members of its last writer, A's first: that group runs paired and
  //    writes the product into the copy the consumer reads (units of two
  //    row-groups only).  When no group writes x, the product is copied
  //    before the step.
  // The first glued group that fits neither ends the persistent part.
  int nkeys = 0;
  if (multi) {
    std::map<std::pair<const void*, int64_t>, int> early_keys;
    size_t cut = groups.size();
    for (size_t g = 0; g < groups.size() && cut == groups.size(); ++g) {
      HostGroup& hg = groups[g];
      if (hg.pro == QD_PRO_NONE) continue;
      const uint64_t xb = (uint64_t)m * hg.k * 2 * (hg.pro == QD_PRO_GLU ? 2 : 1);
      const size_t p = (hg.order & kStageEarly) ? SIZE_MAX : last_writer(groups, g, hg.x, xb, m);
      bool ok = true;
      if (p == SIZE_MAX) {          // no group of the step writes x
        if (hg.pro == QD_PRO_RMSNORM) {
          auto it = early_keys.emplace(std::make_pair((const void*)hg.x, hg.k), nkeys).first;
          if (it->second == nkeys) ++nkeys;
          hg.ss_key = it->second;
          hg.ss_early = true;
        } else {
          hg.glu_src = -2;
        }
      } else if (hg.pro == QD_PRO_RMSNORM) {
        HostGroup& pg = groups[p];
        int q = -1, hits = 0;
        for (size_t b = 0; b < pg.mem.size(); ++b)
          if (ranges_overlap(hg.x, xb, pg.mem[b].y, y_span(pg.mem[b], m))) {
            q = (int)b;
            ++hits;
          }
        ok = hits == 1 && !pg.paired && (const void*)pg.mem[q].y == (const void*)hg.x &&
             pg.mem[q].n == hg.k && pg.mem[q].ld == hg.k;
        for (size_t b = 0; ok && b < pg.mem.size(); ++b)
          if ((int)b != q && pg.rec[b] >= 0) ok = false;
        if (ok) {
          if (pg.rec[q] < 0) pg.rec[q] = nkeys++;
          hg.ss_key = pg.rec[q];
        }
      } else {
        HostGroup& pg = groups[p];
        ok = unit16(fmt) == 2 && pg.mem.size() == 2 && pg.rec[0] < 0 && pg.rec[1] < 0 &&
             (const void*)pg.mem[0].y == (const void*)hg.x &&
             (const void*)pg.mem[1].y == (const void*)(hg.x + m * hg.k) &&
             pg.mem[0].n == hg.k && pg.mem[1].n == hg.k && pg.mem[0].ld == hg.k && pg.mem[1].ld == hg.k &&
             paired_piece(pg.R, pg.J, QD_PLAN_TILES16, G) > 0;
        if (ok) {
          pg.paired = true;
          hg.glu_src = (int64_t)p;
        }
      }
      if (!ok) cut = g;
    }
    if (cut < groups.size()) {
      // The boundary ordering is redone for the groups kept: what the
      // replayed ops read needs no ordering inside the kernel.
      split = groups[cut].src[0];
      groups.resize(cut);
      for (HostGroup& hg : groups) hg.order = 0;
      order_groups(groups, m, tile_bytes(fmt));
    }
  }
  bool glue = false;
  for (const HostGroup& hg : groups) {
    glue = glue || hg.pro != QD_PRO_NONE;
    for (const PMember& pm : hg.mem) glue = glue || pm.epi != QD_EPI_NONE;
  }

  // Several token rows: copies of the activations in matrix-core order.  An
  // activation no group writes is copied before the step; one that is
  // exactly an earlier op's whole output (the last write to any of its
  // bytes) is written in that order by the op itself.  A gated product's copy
  // holds the product (written by the paired group, or made before the
  // step).  Other activations are read in place.
  std::vector<HostJob> jobs;
  int64_t xt_total = 0;
  if (multi && scratch) {
    std::map<std::tuple<const void*, int64_t, int>, int64_t> early_slots;
    std::map<std::pair<size_t, size_t>, int64_t> out_slots;
    auto new_slot = [&](int J) {
      const int64_t off = xt_total;
      xt_total += (int64_t)align_up((size_t)J * 8192, 256);
      return off;
    };
    auto early_slot = [&](const HostGroup& hg, int glu) {
      const auto key = std::make_tuple((const void*)hg.x, hg.k, glu);
      auto it = early_slots.find(key);
      if (it == early_slots.end()) {
        it = early_slots.emplace(key, new_slot(hg.J)).first;
        jobs.push_back(HostJob{hg.x, hg.k, it->second, -1, glu, 0});
      }
      return it->second;
    };
    for (size_t g = 0; g < groups.size(); ++g) {
      HostGroup& hg = groups[g];
      if (hg.pro == QD_PRO_GLU) {
        if (hg.glu_src == -2) {
          hg.xt_off = early_slot(hg, 1);
        } else {
          const size_t p = (size_t)hg.glu_src;
          auto it = out_slots.find(std::make_pair(p, (size_t)0));
          if (it == out_slots.end()) it = out_slots.emplace(std::make_pair(p, (size_t)0), new_slot(hg.J)).first;
          groups[p].yt_off[0] = it->second;
          hg.xt_off = it->second;
        }
        continue;
      }
      if (hg.order & kStageEarly) {
        hg.xt_off = early_slot(hg, 0);
        continue;
      }
      size_t p = SIZE_MAX, q = 0;
      for (size_t j = 0; j < g; ++j)
        for (size_t b = 0; b < groups[j].mem.size(); ++b)
          if (ranges_overlap(hg.x, (uint64_t)m * hg.k * 2, groups[j].mem[b].y, y_span(groups[j].mem[b], m))) {
            p = j;
            q = b;
          }
      if (p == SIZE_MAX || groups[p].paired) continue;   // a paired group's copy slot holds its product
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

  // Sum-of-squares records: G per member slice with records (one per
  // workgroup), in plan order, so that the slices of one op are contiguous;
  // then one per activation summed before the step.
  std::map<int, std::pair<int64_t, int64_t>> recs;   // key -> first record, records
  int64_t ss_total = 0;
  for (HostGroup& hg : groups)
    for (size_t b = 0; b < hg.mem.size(); ++b)
      if (hg.rec[b] >= 0) {
        auto& e = recs[hg.rec[b]];
        if (e.second == 0) e.first = ss_total;
        e.second += G;
        hg.mem[b].ss = (int32_t)ss_total;
        ss_total += G;
      }
  for (HostGroup& hg : groups)
    if (hg.ss_early && !recs.count(hg.ss_key)) {
      recs[hg.ss_key] = std::make_pair(ss_total, (int64_t)1);
      jobs.push_back(HostJob{hg.x, hg.k, -1, ss_total, 0, 0});
      ++ss_total;
    }

  const int ng = (int)groups.size();
  L->pg.resize(ng);
  L->ps.resize((size_t)ng * G);
  std::vector<int32_t> off(G, 0);
  std::vector<int64_t> given(G, 0);  // tiles each workgroup has so far
  int maxJ = 1, maxXH = 512, maxRel = 1, maxSeg = 1, maxGamma = 0;
  int64_t weight_bytes = 0;
  bool any_wait = false;       // some group waits for the one before it
  for (int g = 1; g < ng; ++g) any_wait = any_wait || !(groups[g].order & kNoWait);
  for (int g = 0; g < ng; ++g) {
    HostGroup& hg = groups[g];
    const int64_t J = hg.J, R = hg.R, T = R * J;
    // A step the persistent walker cannot hold (tile counts past int32)
    // replays per-group launches instead.
    if (T > (int64_t)INT32_MAX / 2) return;
    weight_bytes += T * tile_bytes(fmt);
    int32_t ss0 = 0, ss_n = 0;
    if (multi && hg.pro == QD_PRO_RMSNORM) {
      const auto& e = recs.at(hg.ss_key);
      ss0 = (int32_t)e.first;
      ss_n = (int32_t)e.second;
      maxGamma = std::max(maxGamma, x_span(hg.J * kSuperK));
    }
    L->pg[g] = PGroup{hg.x, hg.gamma, nullptr, (int32_t)hg.k, hg.J, hg.R, (int32_t)L->pm.size(),
                      (int32_t)hg.mem.size(), hg.pro, hg.eps, hg.order | (hg.paired ? kPaired : 0), ss0, ss_n};
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
    // than the uneven split.  A paired group is spread in whole pairs.
    //
    // A group whose row-groups do not divide evenly starts its run of
    // ranges at the workgroup (rot) that leaves the lowest largest total of
    // tiles so far (the first such).  With the ranges always in the same
    // place, the same workgroups would take the extra row-groups of every
    // layer (8B-shaped step: q|k|v has 384 row-groups for 256 workgroups, so
    // every other workgroup would carry 16 tiles a layer more, 4% above the
    // mean over the step), and with independent groups the step ends when
    // the most loaded workgroup does.  A group that waits for the one
    // before it starts the totals afresh (every workgroup is level there),
    // so it keeps workgroup order, as paired groups do.
    if (!(hg.order & kNoWait)) std::fill(given.begin(), given.end(), (int64_t)0);
    // One token row, 3 GiB of weights or more: the step's last group, when
    // it has at least four row-groups per workgroup, is split at run time
    // instead (kDynamic).  The workgroups reach it at different times: each
    // streams at its own rate (on the 8B-shaped step the workgroups of some
    // XCDs finish their share 5-8% later than others', the lag adding up
    // over the step), so with a fixed split the early ones would idle while
    // the late ones finish.  Each claims chunks of C row-groups from a device
    // counter as it goes, about 32 per workgroup in all (C = 1 for the 8B
    // and 27B-shaped heads).  Measured, same
    // devices, wall us/step, fixed / dynamic: 8B int8 1259 / 1243, 1302 / 1288,
    // 1298 / 1289 (the last workgroups' finishing times spread 4 us instead
    // of 110); 27B-shaped 3676 / 3672, 3648-3660 / 3652.  With claims of
    // about 16 per workgroup the smaller steps lost what they gained (2B 370
    // / 383, 4B 734-741 / 735-744, 8B INT4 756-764 / 762-777).  (Claims of 8
    // or 4 chunks per workgroup did no better: 8B 1298 / 1304, 2B 374 / 376.)
    // With about 32, single row-groups: 8B 1192-1193 -> 1190, 27B-shaped
    // 3617-3619 -> 3605-3606; and without the stores after the staging and
    // the rings of 2 that go with it for the larger steps (defer), 4B
    // 731-733 -> 725-726 and 8B INT4 739-741 -> 737-740, while the 2B step
    // (1.8 GB) still loses (343-344 -> 345-346), hence 3 GiB.
    // A step in which some group waits for the one before it keeps the fixed
    // split too: every such wait brings the workgroups level again, so no lag
    // builds up for the claims to absorb, and their upkeep in the waits is
    // pure cost (8B chained 1483-1485 -> 1470, glued 1650-1652 -> 1620-1621).
    if (!any_wait && !multi && !hg.paired && g == ng - 1 && R >= 4 * (int64_t)G &&
        weight_bytes >= ((int64_t)3 << 30)) {
      const int64_t Ju = ceil_div(J, (int64_t)ku1(fmt));
      L->dyn_c = (int)std::max<int64_t>(1, R / (32 * (int64_t)G));
      L->dyn_nch = (int)ceil_div(R, (int64_t)L->dyn_c);
      // Claims run dyn_q chunks ahead of the hand-outs, at least 64 tiles (a
      // claim's round trip is a few tiles' time).
      L->dyn_q = (int)ceil_div(64, L->dyn_c * Ju) + 1;
      L->dyn_max = (int)(4 * ceil_div(L->dyn_nch, (int64_t)G)) + L->dyn_q + 8;
      L->dyn_rcap = pow2_at_least(std::max<int64_t>(256, 16 * Ju));
      L->dyn_scap = pow2_at_least(std::max<int64_t>(32, L->dyn_rcap / Ju + 1));
      L->dyn_win = (int)std::min<int64_t>(L->dyn_scap, L->dyn_rcap / Ju);
      L->pg[g].order |= kDynamic;
      L->defer = weight_bytes >= ((int64_t)6 << 30);
      for (int w = 0; w < G; ++w) L->ps[(size_t)g * G + w] = PSched{0, off[w], 0, 0};
      maxRel = std::max(maxRel, L->dyn_rcap);
      maxSeg = std::max(maxSeg, L->dyn_scap);
      continue;
    }
    int rot = 0;
    if (!hg.paired && R % G != 0) {
      int64_t best = INT64_MAX;
      for (int p = 0; p < G; ++p) {
        int64_t top = 0;
        for (int w = 0; w < G; ++w) {
          const int64_t i = (w - p + G) % G;
          top = std::max(top, given[w] + ((i + 1) * R / G - i * R / G) * J);
        }
        if (top < best) {
          best = top;
          rot = p;
        }
      }
    }
    for (int w = 0; w < G; ++w) {
      // Contiguous row-groups: each workgroup streams one contiguous range.
      // (Interleaving them, row-group w + i G to workgroup w, measured 2-11%
      // slower: the contiguous streams keep DRAM pages open.)
      // Several token rows: the sequence holds units of unit16(fmt) row-groups.
      int64_t r0, nrg;
      if (hg.paired) {
        const int64_t P = R / 2;
        r0 = 2 * ((int64_t)w * P / G);
        nrg = 2 * ((int64_t)(w + 1) * P / G) - r0;
      } else {
        const int64_t i = (w - rot + G) % G;
        r0 = i * R / G;
        nrg = (i + 1) * R / G - r0;
      }
      const int64_t n = multi ? ceil_div(nrg, (int64_t)unit16(fmt)) * J : nrg * ceil_div(J, (int64_t)ku1(fmt));
      L->ps[(size_t)g * G + w] = PSched{(int32_t)n, off[w], (int32_t)r0, (int32_t)nrg};
      given[w] += nrg * J;
      if (nrg == 0) continue;
      off[w] += (int32_t)n;
      maxRel = std::max<int>(maxRel, (int)(multi ? nrg * J : n));
      maxSeg = std::max<int>(maxSeg, (int)nrg);
    }
  }
  // One token row: staged activations.  Several: no staged activations,
  // 16 x 16 partials per tile, and under RMSNorm gamma and the 16 per-token
  // factors.
  L->x_bytes = multi ? (size_t)maxGamma * 2 : (size_t)maxXH * 2;      // a multiple of 1024
  L->xsum_bytes = multi ? (maxGamma > 0 ? 64 : 0) : (glue ? 80 : 0);
  L->red_bytes = align_up((size_t)maxRel * 16 * 4 * (multi ? 16 : 1), 16);
  L->cnt_bytes = align_up((size_t)maxSeg * 4, 16);
  L->tab_bytes = (size_t)ng * sizeof(PGroup) + L->pm.size() * sizeof(PMember) + (size_t)ng * sizeof(PSched);
  // + the tile counter and the flags, then the dynamic group's claims
  L->lds = L->x_bytes + L->xsum_bytes + L->red_bytes + L->cnt_bytes + L->tab_bytes + 16 + 16 +
           4 * (size_t)std::max(1, L->dyn_max);
  int64_t blocks = 0;
  for (HostJob& jb : jobs) {
    jb.first_block = blocks;
    blocks += jb.copy_off >= 0 ? 2 * ceil_div(jb.k, kSuperK) : 1;   // 512 chunks per super-block; a record: 1
  }
  L->jobs = std::move(jobs);
  L->xt_total = xt_total;
  L->xt_blocks = blocks;
  L->ss_total = ss_total;
  L->lag = drift_lag(weight_bytes, multi);
  bool waits = false;          // a group that waits for the one before it
  for (size_t g = 1; g < L->pg.size(); ++g) waits = waits || !(L->pg[g].order & kNoWait);
  L->light = !waits;
  L->fmt = fmt;
  L->multi = multi;
  L->glue = glue;
  L->split = split;
  L->persistent = true;
}

}  // namespace

// The dynamic last group's kernel arguments; `ctr`: two zeroed counters.
void set_dynamic(PlanArgs& a, const PlanLayout& L, uint32_t* ctr) {
  a.dyn_ctr = ctr;
  a.dyn_c = L.dyn_c;
  a.dyn_q = L.dyn_q;
  a.dyn_nch = L.dyn_nch;
  a.dyn_max = L.dyn_max;
  a.dyn_rcap = std::max(1, L.dyn_rcap);
  a.dyn_scap = std::max(1, L.dyn_scap);
  a.dyn_win = L.dyn_win;
  a.defer = L.defer ? 1 : 0;
}

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
  const void* kfn = kernel_ptr(L.fmt, L.multi, L.glue, L.light, L.defer);
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

  auto fail = [&]() {
    if (plan->tables) (void)hipFree(plan->tables);
    if (plan->scratch) (void)hipFree(plan->scratch);
    if (plan->xt) (void)hipFree(plan->xt);
    if (plan->xt_jobs) (void)hipFree(plan->xt_jobs);
    delete plan;
    return QD_ELAUNCH;
  };
  // Scratch: the completion stamps, the error word and the sum-of-squares
  // records (zeroed here; every run rewrites the records it reads).
  const size_t s_flags = 0;
  const size_t s_err = align_up(sizeof(unsigned long long) * G, 256);
  const size_t s_ss = s_err + 256;
  const size_t s_bytes = s_ss + align_up((size_t)L.ss_total * 64, 256);
  if (hipMalloc(&plan->scratch, s_bytes) != hipSuccess || hipMemset(plan->scratch, 0, s_bytes) != hipSuccess)
    return fail();
  uint8_t* sb = static_cast<uint8_t*>(plan->scratch);
  float* const ss = L.ss_total > 0 ? reinterpret_cast<float*>(sb + s_ss) : nullptr;

  // The activation copies (zeroed once: token rows past m and K positions
  // past K stay zero) and the table of jobs made before each step.
  if (L.xt_total > 0 &&
      (hipMalloc(&plan->xt, (size_t)L.xt_total) != hipSuccess ||
       hipMemset(plan->xt, 0, (size_t)L.xt_total) != hipSuccess))
    return fail();
  uint8_t* const xb = static_cast<uint8_t*>(plan->xt);
  if (!L.jobs.empty()) {
    std::vector<XtJob> dev_jobs;
    for (const HostJob& jb : L.jobs)
      dev_jobs.push_back(XtJob{jb.x, jb.copy_off >= 0 ? reinterpret_cast<uint16_t*>(xb + jb.copy_off) : nullptr,
                               jb.rec >= 0 ? ss + jb.rec * 16 : nullptr, jb.k, jb.first_block, jb.glu, 0});
    if (hipMalloc(&plan->xt_jobs, sizeof(XtJob) * dev_jobs.size()) != hipSuccess ||
        hipMemcpy(plan->xt_jobs, dev_jobs.data(), sizeof(XtJob) * dev_jobs.size(), hipMemcpyHostToDevice) !=
            hipSuccess)
      return fail();
    plan->xt_njobs = (int)dev_jobs.size();
    plan->xt_blocks = L.xt_blocks;
  }
  for (int g = 0; g < ng; ++g)
    if (L.xt_fix[g] >= 0) pg[g].xt = reinterpret_cast<const uint16_t*>(xb + L.xt_fix[g]);
  for (size_t i = 0; i < pm.size(); ++i)
    if (L.yt_fix[i] >= 0) pm[i].yt = reinterpret_cast<uint16_t*>(xb + L.yt_fix[i]);

  // Device tables.
  const size_t o_groups = 0;
  const size_t o_mem = align_up(o_groups + sizeof(PGroup) * ng, 256);
  const size_t o_sched = align_up(o_mem + sizeof(PMember) * pm.size(), 256);
  const size_t t_bytes = align_up(o_sched + sizeof(PSched) * L.ps.size(), 256);
  std::vector<uint8_t> host(t_bytes, 0);
  memcpy(host.data() + o_groups, pg.data(), sizeof(PGroup) * ng);
  memcpy(host.data() + o_mem, pm.data(), sizeof(PMember) * pm.size());
  memcpy(host.data() + o_sched, L.ps.data(), sizeof(PSched) * L.ps.size());
  if (hipMalloc(&plan->tables, t_bytes) != hipSuccess ||
      hipMemcpy(plan->tables, host.data(), t_bytes, hipMemcpyHostToDevice) != hipSuccess ||
      hipDeviceSynchronize() != hipSuccess)
    return fail();
  uint8_t* tb = static_cast<uint8_t*>(plan->tables);
  PlanArgs& a = plan->args;
  a.groups = reinterpret_cast<const PGroup*>(tb + o_groups);
  a.members = reinterpret_cast<const PMember*>(tb + o_mem);
  a.sched = reinterpret_cast<const PSched*>(tb + o_sched);
  a.flags = reinterpret_cast<unsigned long long*>(sb + s_flags);
  a.err = reinterpret_cast<uint32_t*>(sb + s_err);
  a.ss = ss;
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
  a.lag = L.lag;
  set_dynamic(a, L, reinterpret_cast<uint32_t*>(sb + s_err + 64));   // two counters beside the error word
  plan->scratch_bytes = s_bytes;
  plan->lds = lds;
  plan->fmt = L.fmt;
  plan->multi = L.multi;
  plan->glue = L.glue;
  plan->light = L.light;
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
  std::vector<int64_t> v = {4, L.persistent, L.fmt, m, L.glue, L.persistent ? L.split : 0,
                            (int64_t)L.pg.size(), (int64_t)L.pm.size(), L.G, L.xt_total,
                            (int64_t)L.jobs.size(), (int64_t)L.lds, (int64_t)L.x_bytes,
                            (int64_t)L.red_bytes, (int64_t)L.cnt_bytes, (int64_t)L.tab_bytes, L.ss_total, L.lag,
                            L.dyn_c, L.dyn_q, L.dyn_nch, L.dyn_max};
  auto addr = [](const void* p) { return (int64_t)(uintptr_t)p; };
  for (size_t g = 0; g < L.pg.size(); ++g) {
    const PGroup& p = L.pg[g];
    v.insert(v.end(), {addr(p.x), addr(p.gamma), p.k, p.J, p.R, p.mem0, p.n_mem, p.pro, p.order, L.xt_fix[g],
                       p.ss0, p.ss_n});
  }
  for (size_t i = 0; i < L.pm.size(); ++i) {
    const PMember& p = L.pm[i];
    v.insert(v.end(), {addr(p.blob), addr(p.y), p.n, p.rg_begin, p.epi, p.ld, L.yt_fix[i], p.ss});
  }
  for (const PSched& s : L.ps) v.insert(v.end(), {s.n, s.off, s.rg0, s.nseg});
  for (const HostJob& j : L.jobs) v.insert(v.end(), {addr(j.x), j.copy_off, j.k, j.first_block, j.glu, j.rec});
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
  // One workgroup per CU, each needing a whole CU (1024 threads and most of
  // its LDS), so on an otherwise idle device a plain launch makes them all
  // resident at once; it saves the cooperative launch's own cost (about 30
  // us per step, measured).  Should another kernel hold CUs, some
  // workgroups would wait for it: the first device-wide wait then times out
  // (every wait is bounded, so the kernel still ends), the run reports the
  // timeout, and the plan launches cooperatively from then on.
  const void* kfn = kernel_ptr(plan->fmt, plan->multi, plan->glue, plan->light, plan->args.defer != 0);
  const hipError_t e =
      plan->cooperative
          ? hipLaunchCooperativeKernel(kfn, dim3(plan->args.G), dim3(kWaves * 64), kargs, (unsigned)plan->lds, s)
          : hipLaunchKernel(kfn, dim3(plan->args.G), dim3(kWaves * 64), kargs, (unsigned)plan->lds, s);
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
    // A timed-out wait leaves the counters inconsistent: start over.  The
    // workgroups may not all have been resident (another kernel held CUs):
    // later runs launch cooperatively, which guarantees they are.
    if (hipMemset(plan->scratch, 0, plan->scratch_bytes) != hipSuccess ||
        hipDeviceSynchronize() != hipSuccess)
      return QD_ELAUNCH;
    plan->epoch = 0;
    plan->cooperative = true;
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


// ---------------------------------------------------------------------------
// The persistent step without a plan object, for callers that cannot
// allocate device memory (code under graph capture, serving loops, harnesses
// that forbid hipMalloc).  The plan's tables and scratch live in one static
// device array per device, `scratch`, resolved once per device with
// hipGetSymbolAddress; every call rewrites what it uses:
//   [0, 4096)            completion stamps of up to kMaxWorkgroups workgroups
//   [4096, 4352)         the error word
//   groups, members      the step's group and member tables (at most
//                        kStaticGroups / kStaticMembers records, after the
//                        row-range split at several token rows)
//   schedule             [group][workgroup] records, computed on the device
// The tables reach the device as kernel arguments of small copy kernels, so a
// captured graph replays exactly the call that was captured; nothing is
// copied from host memory that could change afterwards.  Activations are read
// in place (no copies in matrix-core order).  Calls that overlap on one
// device race on the array.

constexpr int kStaticGroups = 512;
constexpr int kStaticMembers = 1024;
constexpr size_t kStaticErrOff = (size_t)kMaxWorkgroups * 8;
constexpr size_t kStaticGroupsOff = kStaticErrOff + 256;
constexpr size_t kStaticMembersOff = kStaticGroupsOff + (size_t)kStaticGroups * sizeof(PGroup);
constexpr size_t kStaticSchedOff = kStaticMembersOff + (size_t)kStaticMembers * sizeof(PMember);
constexpr size_t kStaticBytes = kStaticSchedOff + (size_t)kStaticGroups * kMaxWorkgroups * sizeof(PSched);
static_assert(kStaticGroupsOff % 256 == 0 && kStaticMembersOff % 16 == 0 && kStaticSchedOff % 16 == 0,
              "tables are written in 16-byte units");

// About 4.1 MiB per device, held until the process ends.
static __device__ __align__(256) uint8_t scratch[kStaticBytes];

namespace {

constexpr int kPutBytes = 3072;   // table bytes per copy launch (kernel arguments stay below 4 KiB)
struct PutPayload {
  uint32_t n16;                   // 16-byte units in `data`
  uint32_t pad[3];
  u32x4 data[kPutBytes / 16];
};

__global__ __launch_bounds__(256) void put_kernel(u32x4* __restrict__ dst, PutPayload p) {
  for (uint32_t i = threadIdx.x; i < p.n16; i += 256) dst[i] = p.data[i];
}

// Clear the stamps and the error word, and give each workgroup w its part of
// every group: whole row-groups w R / G .. (w + 1) R / G, in tiles (at several
// token rows, in units of `unit` row-groups), with its running offset in the
// workgroup's sequence (the host's layout_plan computes the same records).
__global__ __launch_bounds__(kMaxWorkgroups) void static_setup_kernel(uint8_t* __restrict__ base, int ngroups,
                                                                      int G, int unit, int ku) {
  const int w = threadIdx.x;
  reinterpret_cast<unsigned long long*>(base)[w] = 0ull;
  if (w == 0) *reinterpret_cast<uint32_t*>(base + kStaticErrOff) = 0u;
  if (w < 2) reinterpret_cast<uint32_t*>(base + kStaticErrOff + 64)[w] = 0u;   // the claim counters
  if (w >= G) return;
  const PGroup* gs = reinterpret_cast<const PGroup*>(base + kStaticGroupsOff);
  PSched* sched = reinterpret_cast<PSched*>(base + kStaticSchedOff);
  int32_t off = 0;
  for (int g = 0; g < ngroups; ++g) {
    const int64_t R = gs[g].R, J = gs[g].J;
    const int64_t r0 = (int64_t)w * R / G, nrg = (int64_t)(w + 1) * R / G - r0;
    if (gs[g].order & kDynamic) {                   // split at run time
      sched[(size_t)g * G + w] = PSched{0, off, 0, 0};
      continue;
    }
    const int64_t n = unit > 1 ? (nrg + unit - 1) / unit * J : nrg * ((J + ku - 1) / ku);
    sched[(size_t)g * G + w] = PSched{(int32_t)n, off, (int32_t)r0, (int32_t)nrg};
    if (nrg != 0) off += (int32_t)n;
  }
}

__global__ void static_report_kernel(const uint32_t* __restrict__ err, int32_t* __restrict__ out) {
  if (threadIdx.x == 0 && *err != 0u) atomicOr(out, (int32_t)*err);
}

struct StaticDevice {
  bool ready = false;
  hipError_t status = hipSuccess;
  uint8_t* base = nullptr;        // device address of `scratch` on this device
  int cus = 0;
  size_t lds_max = 0;
};

constexpr int kStaticDevices = 64;
std::mutex g_static_mu;
StaticDevice g_static[kStaticDevices];

// Set-up, once per device (with that device current): the array's device
// address and the device's compute units and LDS.
const StaticDevice* static_device(int dev) {
  if (dev < 0 || dev >= kStaticDevices) return nullptr;
  std::lock_guard<std::mutex> lock(g_static_mu);
  StaticDevice& d = g_static[dev];
  if (!d.ready) {
    d.ready = true;
    void* ptr = nullptr;
    d.status = hipGetSymbolAddress(&ptr, HIP_SYMBOL(scratch));
    hipDeviceProp_t prop;
    if (d.status == hipSuccess) d.status = hipGetDeviceProperties(&prop, dev);
    if (d.status == hipSuccess) {
      d.base = static_cast<uint8_t*>(ptr);
      d.cus = prop.multiProcessorCount;
      d.lds_max = std::max<size_t>(prop.sharedMemPerBlock, prop.maxSharedMemoryPerMultiProcessor);
    } else {
      (void)hipGetLastError();
    }
  }
  return d.status == hipSuccess ? &d : nullptr;
}

hipError_t put_table(uint8_t* dst, const void* src, size_t bytes, hipStream_t s) {
  const uint8_t* p = static_cast<const uint8_t*>(src);
  for (size_t done = 0; done < bytes; done += kPutBytes) {
    PutPayload pl{};
    const size_t n = std::min<size_t>(kPutBytes, bytes - done);
    pl.n16 = (uint32_t)((n + 15) / 16);
    memcpy(pl.data, p + done, n);
    hipLaunchKernelGGL(put_kernel, dim3(1), dim3(256), 0, s, reinterpret_cast<u32x4*>(dst + done), pl);
    const hipError_t e = hipGetLastError();
    if (e != hipSuccess) return e;
  }
  return hipSuccess;
}

}  // namespace

qd_status stack_run_noalloc(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t* err_flag, hipStream_t s) {
  std::vector<StackGroup> replay;
  qd_status st = build_groups(ops, n_ops, m, &replay);
  if (st != QD_OK) return st;
  if (err_flag && (uintptr_t)err_flag % 4) return QD_EALIGN;
  int dev = 0;
  if (hipGetDevice(&dev) != hipSuccess) return QD_EDEVICE;
  const StaticDevice* sd = static_device(dev);
  if (!sd) return QD_EDEVICE;
  const int G = std::min(sd->cus, kMaxWorkgroups);
  PlanLayout L;
  layout_plan(ops, n_ops, m, G, &L, /*scratch=*/false);
  auto replay_all = [&]() { return launch_groups(replay, s) == hipSuccess ? QD_OK : QD_ELAUNCH; };
  if (!L.persistent) return replay_all();
  if (L.pg.size() > (size_t)kStaticGroups || L.pm.size() > (size_t)kStaticMembers) return QD_ESHAPE;
  std::vector<StackGroup> tail;
  if (L.split < n_ops && build_groups(ops + L.split, n_ops - L.split, m, &tail) != QD_OK) return replay_all();
  const void* kfn = kernel_ptr(L.fmt, L.multi, L.glue, L.light, L.defer);
  if (L.lds > sd->lds_max) return replay_all();
  if (L.lds > 65536 && hipFuncSetAttribute(kfn, hipFuncAttributeMaxDynamicSharedMemorySize, (int)L.lds) != hipSuccess) {
    (void)hipGetLastError();
    return replay_all();
  }
  int per_cu = 0;
  if (hipOccupancyMaxActiveBlocksPerMultiprocessor(&per_cu, kfn, kWaves * 64, L.lds) != hipSuccess || per_cu < 1) {
    (void)hipGetLastError();
    return replay_all();
  }
  uint8_t* const base = sd->base;
  if (put_table(base + kStaticGroupsOff, L.pg.data(), sizeof(PGroup) * L.pg.size(), s) != hipSuccess ||
      put_table(base + kStaticMembersOff, L.pm.data(), sizeof(PMember) * L.pm.size(), s) != hipSuccess)
    return QD_ELAUNCH;
  hipLaunchKernelGGL(static_setup_kernel, dim3(1), dim3(kMaxWorkgroups), 0, s, base, (int)L.pg.size(), G,
                     L.multi ? unit16(L.fmt) : 1, L.multi ? 1 : ku1(L.fmt));
  if (hipGetLastError() != hipSuccess) return QD_ELAUNCH;
  PlanArgs a{};
  a.groups = reinterpret_cast<const PGroup*>(base + kStaticGroupsOff);
  a.members = reinterpret_cast<const PMember*>(base + kStaticMembersOff);
  a.sched = reinterpret_cast<const PSched*>(base + kStaticSchedOff);
  a.flags = reinterpret_cast<unsigned long long*>(base);
  a.err = reinterpret_cast<uint32_t*>(base + kStaticErrOff);
  a.epoch = 1;                    // stamps were cleared above
  a.ngroups = (int32_t)L.pg.size();
  a.nmem = (int32_t)L.pm.size();
  a.G = G;
  a.x_bytes = (int32_t)L.x_bytes;
  a.xsum_bytes = (int32_t)L.xsum_bytes;
  a.red_bytes = (int32_t)L.red_bytes;
  a.cnt_bytes = (int32_t)L.cnt_bytes;
  a.tab_bytes = (int32_t)L.tab_bytes;
  a.m = (int32_t)m;
  a.spin_limit = kSpinLimit;
  a.lag = L.lag;
  set_dynamic(a, L, reinterpret_cast<uint32_t*>(base + kStaticErrOff + 64));
  void* kargs[] = {&a};
  // A plain launch, as a plan's: capturable in a graph.
  if (hipLaunchKernel(kfn, dim3(G), dim3(kWaves * 64), kargs, (unsigned)L.lds, s) != hipSuccess) return QD_ELAUNCH;
  if (err_flag) {
    hipLaunchKernelGGL(static_report_kernel, dim3(1), dim3(64), 0, s, a.err, err_flag);
    if (hipGetLastError() != hipSuccess) return QD_ELAUNCH;
  }
  if (!tail.empty() && launch_groups(tail, s) != hipSuccess) return QD_ELAUNCH;
  return QD_OK;
}

}  // namespace qd
