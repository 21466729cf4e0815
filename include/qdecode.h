/*
 * qdecode -- weight-only quantized linear layers for LLM decoding on
 * AMD Instinct MI355X (gfx950).  C ABI.
 *
 * What is computed
 *   y = W^ x for an fp16 activation vector x (one decoded token), or
 *   Y = X W^T for up to 16 token rows (a static chunked-prefill step), where
 *   W^ is a weight matrix stored quantized:
 *
 *   int8 b32  -- int8 codes, symmetric absmax per block of 32 consecutive
 *                weights along K, one fp16 scale per block: s = fp16(fl32(
 *                max|w| / 127)), q = clamp(rint(fl32(w / s)), -127, 127),
 *                w^ = q s.  The pages call this the "int8 per-block-32 body +
 *                untied absmax int8 head" ship config (Qwen3-VL 4B/8B Core AI
 *                cards, Files table; zoo Qwen3-VL page, Measured paragraph) and
 *                apply the same absmax rule to the LM head without clipping
 *                (zoo Qwen3.8-27B page, Numerics paragraph).
 *   int4 g64  -- 4-bit codes per group of 64 along K (CoreML-LLM Qwen3-VL
 *                4B/8B handoff page, Architecture paragraph), in affine form:
 *                s = fp16(fl32(fl32(max - min) / 15)), m = fp16(min),
 *                q = clamp(rint(fl32(fl32(w - m) / s)), 0, 15), w^ = m + q s;
 *                min and max order -0 below +0 (IEEE 754-2019 minimum and
 *                maximum), so a group whose least value is zero stores the min
 *                -0 when any of its zeros is -0.
 *   A zero scale gives zero codes.  Rounding is IEEE round-to-nearest-even
 *   throughout.
 *
 *   Decode is bandwidth-bound: each step streams every quantized weight once
 *   (Core AI 4B/8B cards, Measured paragraph).  The kernels read each packed
 *   byte exactly once per call and dequantize in registers.
 *
 * Conventions
 *   - Matrices are [N, K] row-major in the PyTorch Linear sense: y[n] =
 *     sum_k W[n,k] x[k].  fp16 values travel as uint16_t bit patterns.
 *   - Every data pointer is a DEVICE pointer unless marked "host".  The caller
 *     owns every buffer; the library never allocates on the compute path
 *     (only qd_stack_plan_create allocates, once).
 *   - `stream` is a hipStream_t (NULL = the default stream).  Calls validate
 *     their arguments on the host and return synchronously; on success the
 *     work is enqueued on `stream` and runs asynchronously.  On any error
 *     nothing is enqueued.  Errors raised while a kernel runs surface at the
 *     next synchronizing HIP call.
 *   - An op's output must not overlap its own inputs (x, gamma, weights).  In
 *     a stack, the outputs of one group must not overlap each other; a later
 *     group may read or overwrite an earlier group's buffers.
 *   - The functions hold no global mutable state and are thread-safe, except
 *     that one qd_stack_plan must not run on two streams at once.
 *
 * Packed layout ("tiled blob")
 *   Rows are padded to Np = 16 ceil(N/16), K to Kp = 256 ceil(K/256), with
 *   zero codes, scales and mins.  Row-group r = rows 16r..16r+15; super-block
 *   j = k in [256j, 256j+256).  Tile (r, j) starts at byte (r (Kp/256) + j) T.
 *   In each 1024-byte chunk of a tile, lane l = 16g + rho (0..63) owns bytes
 *   16l..16l+15 for row 16r + rho and K-quarter g.
 *   int8 b32, T = 4352: chunk s = 0..3; lane bytes 0..7 = codes at k = 256j +
 *     64s + 8g + i, bytes 8..15 = codes at k = 256j + 64s + 32 + 8g + i
 *     (i = 0..7); then 16 rows x 8 fp16 scales (blocks 8j..8j+7) at 4096 +
 *     16 rho.
 *   int4 g64, T = 2304: chunk s = 0..1; lane bytes 0..7 = codes of group
 *     4j+2s, in-group offsets 16g..16g+15; bytes 8..15 = same for group
 *     4j+2s+1; each little-endian uint32 holds 8 consecutive codes k0..k0+7
 *     with nibble p holding code k0 + (0,2,4,6,1,3,5,7)[p]; then per row rho
 *     at 2048 + 16 rho: 4 fp16 scales, 4 fp16 mins (groups 4j..4j+3).
 *   fp16, T = 8192: chunk s = 0..7; lane bytes 0..15 = the fp16 weights at
 *     k = 256j + 32s + 8g + i (i = 0..7).
 *   With N % 16 == 0 and K % 256 == 0 the blob holds exactly N K (1 + 2/32)
 *   (int8), N K (1/2 + 4/64) (int4) or 2 N K (fp16) bytes.
 *
 * Formats
 *   int8 b32 and INT4 g64 as defined with their packers below.  fp16 is the
 *   unquantized head of the pages' int8lin variant (zoo Qwen3-VL page,
 *   Measured table, "2B int8lin (tied fp16 head)" row): w^ = fp16_RNE(w).
 */
#ifndef QDECODE_H
#define QDECODE_H

#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
  QD_OK = 0,
  QD_EINVAL = 1,   /* null pointer, unknown enum, overlapping buffers, bad plan */
  QD_ESHAPE = 2,   /* K not a multiple of 32 (int8, fp16) / 64 (int4), N or K < 0,
                      K > QD_MAX_K, M outside 1..16, blob smaller than needed */
  QD_EALIGN = 3,   /* blob, x, gamma or W not 16-byte aligned */
  QD_ERANGE = 4,   /* (reported through the packer's device flag, see below) */
  QD_ELAUNCH = 5,  /* a HIP launch or runtime call failed */
  QD_EFORMAT = 6,  /* weight format not supported by this entry point */
  QD_EDEVICE = 7   /* no usable device, or the plan belongs to another device */
} qd_status;

typedef enum { QD_FMT_INT8_B32 = 1, QD_FMT_INT4_G64 = 2, QD_FMT_FP16 = 3 } qd_format;

enum { QD_MAX_K = 24576, QD_MAX_M = 16 };

/* A packed weight.  `data` is a device pointer to the tiled blob (16-byte
 * aligned, at least qd_packed_bytes(fmt, n, k) bytes), owned by the caller. */
typedef struct {
  int32_t fmt;        /* qd_format */
  int32_t reserved;   /* 0 */
  int64_t n, k;       /* logical shape [N, K] */
  const void* data;
  uint64_t bytes;     /* size of the buffer at `data` */
} qd_weight;

/* Bytes of the tiled blob for an [n, k] matrix; 0 if the shape is invalid.
 * Host only, pure. */
uint64_t qd_packed_bytes(int32_t fmt, int64_t n, int64_t k);

/* Static description of a status code (host, never NULL). */
const char* qd_status_string(int32_t status);

/*
 * Quantize and pack an fp32 matrix (device, [n, k] row-major, 16-byte
 * aligned) into `out` (device, out_bytes >= qd_packed_bytes).  Bit-exact with
 * the definitions above, including the padding.  A block/group holding a
 * non-finite weight sets bit 1 of *err_flag, one whose scale or min overflows
 * fp16 sets bit 2 (err_flag: device int32, may be NULL; bits are OR-ed in,
 * never cleared); such a block/group is written as zero codes, zero scale.
 * int8: k % 32 == 0.  int4: k % 64 == 0.
 * qpack_fp16 rounds each weight to fp16 (nearest, ties to even); 8 consecutive
 * weights holding a non-finite value set bit 1, a value that rounds beyond
 * the fp16 range sets bit 2, and are written as zeros.  k % 32 == 0.
 */
qd_status qpack_int8_b32(const float* w, int64_t n, int64_t k, void* out, uint64_t out_bytes,
                         int32_t* err_flag, void* stream);
qd_status qpack_int4_g64(const float* w, int64_t n, int64_t k, void* out, uint64_t out_bytes,
                         int32_t* err_flag, void* stream);
qd_status qpack_fp16(const float* w, int64_t n, int64_t k, void* out, uint64_t out_bytes,
                     int32_t* err_flag, void* stream);

/*
 * One decoded token: y[n] = fp16_RNE(sum_k w^[n,k] x[k]) with fp32
 * accumulation.  `w` is a host pointer to the descriptor; x (device, fp16
 * [K], 16-byte aligned) and y (device, fp16 [N]).  N == 0 is a no-op; K == 0
 * writes zeros.  The format must match the entry point (else QD_EFORMAT).
 */
qd_status qgemv_int8_b32(const qd_weight* w, const uint16_t* x, uint16_t* y, void* stream);
qd_status qgemv_int4_g64(const qd_weight* w, const uint16_t* x, uint16_t* y, void* stream);
qd_status qgemv_fp16(const qd_weight* w, const uint16_t* x, uint16_t* y, void* stream);

/*
 * A static chunk of m tokens (1 <= m <= 16, the pages' S=16 chunked-prefill
 * function, zoo Qwen3.8-27B page, vision path section): Y[i, n] =
 * fp16_RNE(sum_k X[i,k] w^[n,k]), X fp16 [m, K] row-major (16-byte aligned),
 * Y fp16 [m, N] row-major.  The contraction runs on the matrix cores.
 * Formats: int8 b32, INT4 g64 and fp16 (the format is taken from the descriptor).
 */
qd_status qgemm_small_m(const qd_weight* w, const uint16_t* x, uint16_t* y, int64_t m, void* stream);

/*
 * Glue fused into a stack op (zoo Qwen3-VL page, Architecture paragraph: a
 * Qwen3 decoder, whose projections are fed by an RMSNorm (q|k|v, gate|up) and
 * by the SwiGLU of the gate and up outputs (down)).  The pages print neither
 * formula; the readings are an fp16 model's, with fp32 arithmetic inside:
 *
 * Prologue (how the op's x becomes the vector it multiplies), per token:
 *   QD_PRO_NONE     x itself.
 *   QD_PRO_RMSNORM  u_k = fp16(gamma_k * fp16(x_k * r)), r = 1 / sqrt(mean_k
 *                   x_k^2 + eps), the mean over the op's K.  `gamma` is fp16
 *                   [K] (device, 16-byte aligned), eps finite and > 0.
 *   QD_PRO_GLU      x holds two fp16 blocks of m x K values, A then B
 *                   (A = x[0 .. mK), B = x[mK .. 2mK), rows of m tokens), and
 *                   u = fp16(A * B) element-wise (one correctly rounded
 *                   product).  With A the gate output under QD_EPI_SILU and B
 *                   the up output this is the SwiGLU h = fp16(fp16(silu(gate))
 *                   * up): point the up op's y at the gate op's y + m * K.
 * Epilogue (what the op stores):
 *   QD_EPI_NONE     y = fp16(W^ u).
 *   QD_EPI_SILU     y = fp16(silu(fp16(W^ u))), silu(a) = a / (1 + e^-a).
 */
typedef enum { QD_PRO_NONE = 0, QD_PRO_RMSNORM = 1, QD_PRO_GLU = 2 } qd_prologue;
typedef enum { QD_EPI_NONE = 0, QD_EPI_SILU = 1 } qd_epilogue;

/*
 * One decode step's linear layers, issued back to back on one stream.
 * ops[i] computes ops[i].y = W^_i ops[i].x (m token rows), with the op's
 * prologue and epilogue.  Consecutive ops with equal `group` form one group:
 * they must share x, K, format and prologue (with its gamma and eps) and are
 * fused into one launch; the epilogue is per op.  Group g+1 starts only after
 * group g has written all its outputs, so a later op's x may be an earlier
 * group's y (a dependent chain).  All ops use the same m (1..16, any format).
 * A prologue other than QD_PRO_NONE, or an unknown epilogue, on an op whose
 * gamma or eps do not match it is QD_EINVAL (gamma must be NULL and eps 0
 * unless the prologue is QD_PRO_RMSNORM); so is x overlapping any op's y in
 * its own group.
 */
typedef struct {
  qd_weight w;
  const uint16_t* x;      /* fp16 [m, K]; [2, m, K] under QD_PRO_GLU */
  uint16_t* y;            /* fp16 [m, N] */
  int32_t group;
  int32_t prologue;       /* qd_prologue */
  const uint16_t* gamma;  /* QD_PRO_RMSNORM weight, fp16 [K]; else NULL */
  float eps;              /* QD_PRO_RMSNORM epsilon; else 0 */
  int32_t epilogue;       /* qd_epilogue */
} qd_linear_op;

qd_status decode_linear_stack(const qd_linear_op* ops, int64_t n_ops, int64_t m, void* stream);

/*
 * The same step as a persistent plan: one kernel launch per step that walks
 * every group in order, keeping the weight stream going across group
 * boundaries (weights of later groups are fetched while a group completes).
 * A group that reads an earlier group's output, or writes what an earlier
 * group reads or writes, starts its products only after every workgroup has
 * finished the group before it; a group independent of every earlier one
 * does not wait for them (outputs are the same either way).  The plan orders
 * each boundary from the step's buffers:
 * a group's activations are read ahead of that barrier only when no earlier
 * group writes any byte of them, and a group's outputs are made visible
 * before its completion is signalled only when a later group reads or
 * rewrites them.  A step computes what decode_linear_stack's sequential
 * launches compute, so an op may consume (or overwrite) an earlier op's
 * buffers; the persistent kernel sums each row's tiles in its own fixed order,
 * so its outputs may differ from the launches' in the last bit (and are the
 * same from run to run).
 * The persistent kernel runs one workgroup per compute unit and needs all of
 * them resident at once.  Runs use a plain launch, which on a device with no
 * other work running makes them so; if another kernel holds compute units,
 * the first device-wide wait of the run times out (waits are bounded, so the
 * kernel still ends), qd_stack_plan_error reports it, and from then on the
 * plan uses a cooperative launch, which guarantees co-residency at a cost of
 * about 30 us per step.
 * qd_stack_plan_create validates `ops` exactly as decode_linear_stack does,
 * copies the descriptors to the device and allocates the plan's scratch
 * (completion stamps, an error word and, at m > 1, copies of the step's
 * activations in the order the matrix cores read them: 8 KiB per 256 input
 * features per group, about 28 MB for an 8B-shaped step, and 64 bytes of
 * RMSNorm statistics per workgroup per op that feeds an RMSNorm) once; the
 * pointers in `ops` must stay valid while the plan lives.
 * qd_stack_plan_run enqueues one step on `stream` (at m > 1 a small kernel
 * for what the step needs of the activations no op of it writes: their
 * copies, gated products and RMSNorm statistics; then the persistent kernel)
 * and allocates nothing.  A plan may be run repeatedly but not
 * concurrently.  The persistent kernel takes groups of one format, int8
 * b32 or INT4 g64, at m = 1..16, with or without glue.  At m > 1 a glued
 * group qualifies when its input is one the kernel can prepare: under
 * QD_PRO_RMSNORM, x is not written by the step, or is exactly the whole
 * output of one op of the last group writing it (that op's workgroups then
 * write per-token sums of squares of what they store, added in a fixed order
 * by the consumer; such an op must be the only one of its group feeding an
 * RMSNorm); under QD_PRO_GLU, x is not written by the step, or its two
 * blocks are exactly the whole outputs of the two ops of the last group
 * writing it, A's first (that group then computes row-group i of both ops
 * together and writes the product itself; it may not also feed an RMSNorm).
 * The plan runs the step's leading groups that qualify; from the first
 * group that does not (say an fp16 head), the rest of the step is replayed
 * after it as the same per-group launches decode_linear_stack makes.  A
 * step whose first group does not qualify (fp16 weights), or whose schedule
 * is larger than one CU's LDS or has a row-group too long for it at m > 1,
 * is replayed whole, with the same results as decode_linear_stack;
 * qd_stack_plan_is_persistent tells whether the persistent kernel runs.
 */
typedef struct qd_stack_plan qd_stack_plan;

qd_status qd_stack_plan_create(const qd_linear_op* ops, int64_t n_ops, int64_t m, qd_stack_plan** out);
qd_status qd_stack_plan_run(qd_stack_plan* plan, void* stream);
/* Device error word of the last completed run (host reads it with a blocking
 * copy): 0 = fine, nonzero = a bounded wait timed out (the step's outputs are
 * incomplete; the plan resets its scratch, switches to cooperative launches
 * and can be run again). */
qd_status qd_stack_plan_error(qd_stack_plan* plan, int32_t* out_error);
/* *out = 1 if runs use the persistent kernel, 0 if they replay launches. */
qd_status qd_stack_plan_is_persistent(const qd_stack_plan* plan, int32_t* out);
/* Diagnostics (not part of the method): bound every wait of the persistent
 * kernel by `polls` polls (default 2^20, about a second) for the following
 * runs.  A small bound makes waits time out, which exercises the error word:
 * such a run's outputs are incomplete and qd_stack_plan_error reports it.
 * No effect on plans that replay launches.  QD_EINVAL for a null plan. */
qd_status qd_stack_plan_set_spin_limit(qd_stack_plan* plan, uint32_t polls);
/* Diagnostics (not part of the method): the schedule qd_stack_plan_create
 * would build for `ops` on a device of `workgroups` compute units, computed
 * on the host alone (no device call; the pointers in `ops` are only compared
 * and offset, never dereferenced, so any values that pass the validation of
 * decode_linear_stack will do).  Writes int64 words to `out` (host memory,
 * caller-owned) and their count to *out_len:
 *   header, 22 words: version (4), persistent (0/1), format, m, glue (0/1),
 *     prefix ops (ops [0, prefix) run in the persistent kernel, the rest are
 *     replayed after it), groups G_n, members M_n, workgroups W, bytes of the
 *     activation copies, pre-step jobs J_n, dynamic LDS bytes, then LDS bytes
 *     of the staged activations (at m > 1: RMSNorm gamma), the tile partials,
 *     the row-group counters and the schedule tables, the number of
 *     RMSNorm statistics records (16 floats each), the drift bound: before
 *     a group independent of every earlier one, how many groups the slowest
 *     workgroup may trail (0: unbounded), and for a last group split at run
 *     time (flag 64 below; else zeros): row-groups per claimed chunk, chunks
 *     claimed ahead of the tile hand-out, chunks in the group and the most
 *     one workgroup may claim;
 *   G_n groups of 12 words, in the order the kernel runs them: x, gamma, K,
 *     super-blocks J, row-groups R, first member, members, prologue, order
 *     flags (1 = may stage early, 2 = acknowledges its stores before its
 *     stamp, 4 = waits for nothing (a later row range of a split group),
 *     8 = reads its activations through the caches, 32 = independent of
 *     every earlier group (reads nothing an earlier group writes, writes
 *     nothing an earlier group reads or writes; also carries 4), 16 = paired: row-group
 *     2i + b is row-group i of member b, and the group writes the gated
 *     product of its two members' outputs, 64 = m = 1, the step's last group
 *     with at least 4 W row-groups: not split in advance (its schedule
 *     entries are zeros); workgroups claim chunks of its row-groups from a
 *     device counter as they reach it), offset of its activation copy in
 *     the plan's copies or -1 (under QD_PRO_GLU at m > 1: of the product),
 *     first statistics record of its RMSNorm input and their count (0, 0
 *     when none);
 *   M_n members of 8 words: weight blob, y, rows N, first row-group within
 *     the group, epilogue, elements between token rows of y, offset of the
 *     copy of its outputs or -1 (a paired group's first member: where it
 *     writes the product), first of its W statistics records or -1;
 *   G_n x W schedule entries of 4 words, group-major: tiles, tiles of this
 *     workgroup in earlier groups, first row-group, row-groups;
 *   J_n pre-step jobs of 6 words: x, offset of its copy or -1, K, first
 *     block, 1 if the copy holds the gated product of x's two blocks, the
 *     statistics record it writes or -1.
 * A step that replays whole gives the header alone.  With out NULL only
 * *out_len is set (a size query, QD_OK); with cap below the count *out_len is
 * set, nothing is written and the result is QD_ESHAPE.  QD_EINVAL for a null out_len, a
 * negative cap or workgroups outside 1..512; otherwise the status
 * decode_linear_stack's validation gives. */
qd_status qd_stack_plan_describe(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t workgroups,
                                 int64_t* out, int64_t cap, int64_t* out_len);
void qd_stack_plan_destroy(qd_stack_plan* plan);

/*
 * For callers that cannot allocate device memory (code under HIP graph
 * capture, tight serving loops, harnesses that forbid hipMalloc): one step of
 * `ops` in the persistent kernel, as a plan made from the same ops would run
 * it, with no plan object and no allocation.  The plan's tables and scratch
 * live in one static device array of about 4.1 MiB per device (held until
 * the process ends), whose address is looked up once per device on the first
 * call; each call rewrites what it uses through small kernels on `stream`
 * (the tables travel as kernel arguments, so a captured graph replays exactly
 * the captured call).  Differences from a plan: activations are always read
 * in place (no copies in matrix-core order, so steps with several token rows
 * run somewhat slower), and at m > 1 the first group with glue ends the
 * persistent part (glue there needs the plan's copies and statistics); the
 * launch is always a plain one (see the plan's launch above; there is no
 * plan to switch to cooperative launches).
 * Arguments and validation as decode_linear_stack; additionally QD_ESHAPE if
 * the step needs more than 512 group records or 1024 member records after
 * the row-range split at several token rows, QD_EALIGN if err_flag is not
 * 4-byte aligned.  `err_flag` (device int32, may be NULL) has the run's
 * error bits OR-ed in (nonzero: a bounded wait timed out; the outputs are
 * incomplete).  Steps the persistent kernel does not take are replayed as
 * decode_linear_stack's launches, as a plan would.  All calls on one device
 * share the array: calls that overlap in time on one device (two streams,
 * two threads) race and must be serialised by the caller.
 */
qd_status qd_stack_run_noalloc(const qd_linear_op* ops, int64_t n_ops, int64_t m, int32_t* err_flag,
                               void* stream);

/*
 * Measurement helper (not part of the method): read every byte of the device
 * buffer `buf` (16-byte aligned, `bytes` > 0) once with a plain streaming
 * kernel of `grid` workgroups (1..65535) x 256 threads, so a run can quote
 * the step's bandwidth as a fraction of what a bare read reaches on this
 * device.  `sink` (device, 4 bytes, 4-byte aligned) is written only if an
 * impossible value turns up; it keeps the loads from being optimised away.
 * Errors: QD_EINVAL (null), QD_EALIGN, QD_ESHAPE (bytes == 0 or grid out of
 * range), QD_ELAUNCH.
 */
qd_status qd_read_probe(const void* buf, uint64_t bytes, void* sink, int32_t grid, void* stream);

#ifdef __cplusplus
}
#endif

#endif /* QDECODE_H */
