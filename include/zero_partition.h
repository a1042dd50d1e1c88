/*
 * zero_partition.h -- C ABI of libzero_partition.so: one rank's share of a
 * ZeRO-DP optimizer step on an MI355X (gfx950).
 *
 * The method is described on the ZeRO explainer page ("ZeRO: Memory
 * Optimizations Toward Training Trillion Parameter Models", azimuth.plus):
 *   - model-states paragraph: per parameter the model states are an fp16
 *     parameter (2 bytes), an fp16 gradient (2 bytes) and an fp32 Adam state
 *     of master copy, momentum and variance (12 bytes), 16 bytes in all;
 *   - Stage 1 (P_os), Stage 2 (P_os+g) and Stage 3 (P_os+g+p) paragraphs:
 *     which of those kinds each of the N ranks keeps only 1/N of, that a
 *     rank reduces only its own gradient slice (reduce-scatter), updates only
 *     its own partition, and that the updated fp16 parameters are gathered
 *     from every rank afterwards;
 *   - constant-size buffers paragraph (ZeRO-R): small tensors are fused into
 *     one fixed-size buffer that does not grow with the model.
 *
 * Conventions
 *   - Every function returns ZERO_OK (0) or a negative zero_status.  A
 *     thread-local message for the last error is in zero_last_error().
 *   - Arguments are checked before anything is launched or written; on an
 *     argument error no host or device state is modified.  After a
 *     ZERO_ERR_HIP the device state reached by the failed call is undefined.
 *   - fp16 values cross the ABI as uint16_t bit patterns (IEEE binary16).
 *   - "device" pointers point into GPU memory of the current HIP device;
 *     "host" pointers into ordinary host memory.  The caller owns every
 *     buffer it passes; the library keeps no pointer beyond the call except
 *     the tensor tables given to zero_layout_bind_tensors and
 *     zero_layout_bind_contributions.
 *   - `stream` is a hipStream_t passed as void* (NULL = the null stream).
 *     Device work is ordered on that stream, which must belong to the
 *     current device (a stream of another device is a STATE error).
 *   - Flat indices and sizes are int64_t.
 */
#ifndef ZERO_PARTITION_H
#define ZERO_PARTITION_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ZERO_PARTITION_VERSION 10000 /* 1.0.0 */

typedef enum zero_status {
    ZERO_OK = 0,
    ZERO_ERR_INVALID_ARG = -1,    /* a null pointer, a size or index out of range */
    ZERO_ERR_ALIGNMENT = -2,      /* a device pointer lacks the required alignment */
    ZERO_ERR_CAPACITY = -3,       /* an output array is too small; the needed count is reported */
    ZERO_ERR_INDEX_OVERFLOW = -4, /* a size or byte count does not fit in int64 */
    ZERO_ERR_HIP = -5,            /* a HIP runtime call failed; see zero_last_hip_error() */
    ZERO_ERR_OUT_OF_MEMORY = -6,  /* host or device allocation failed, or a table would be too large */
    ZERO_ERR_STATE = -7           /* call not valid in this state (e.g. pack before bind) */
} zero_status;

/* ------------------------------------------------------------------------ */
/* Partition layout (host only; no device work)                             */
/* ------------------------------------------------------------------------ */

/* Opaque layout handle, created by zero_partition_layout and freed by
 * zero_layout_destroy. */
typedef struct zero_layout zero_layout;

/* Summary of a layout.  Per-rank byte counts follow the model-states
 * paragraph (2 + 2 + 4 + 4 + 4 bytes per element) and the stage paragraphs:
 *   stage 0  nothing partitioned (plain data parallelism): every kind over Psi
 *   stage 1  master, momentum, variance over S; fp16 param and grad over Psi
 *   stage 2  additionally the fp16 gradient over S
 *   stage 3  additionally the fp16 parameter over S
 * Replicated kinds count the unpadded Psi, partitioned kinds the padded S. */
typedef struct zero_layout_info {
    int64_t psi;             /* total elements, sum of numel */
    int64_t shard_elems;     /* S = roundup(ceil(psi / n_ranks), align_elems) */
    int64_t padded_elems;    /* n_ranks * S */
    int64_t padding;         /* padded_elems - psi */
    int64_t n_tensors;
    int64_t align_elems;
    int64_t bucket_elems;    /* B; 0 when no bucket plan */
    int64_t n_fills;         /* ceil(psi / B); 0 when B == 0 */
    int64_t n_segments;
    int32_t n_ranks;
    int32_t stage;
    int64_t bytes_param16;   /* per-rank bytes of each kind at this stage */
    int64_t bytes_grad16;
    int64_t bytes_master;
    int64_t bytes_momentum;
    int64_t bytes_variance;
    int64_t bytes_total;
} zero_layout_info;

/* One piece of a tensor that lies inside one shard (and, with a bucket plan,
 * inside one bucket fill).  Segments are sorted by flat_off and tile
 * [0, psi) exactly; zero-sized tensors have no segment. */
typedef struct zero_segment {
    int32_t tensor;      /* index in the tensor list */
    int32_t owner;       /* rank owning this piece: flat_off / S */
    int64_t tensor_off;  /* element offset inside the tensor */
    int64_t flat_off;    /* element offset in the flattened vector */
    int64_t len;         /* elements, > 0 */
    int64_t shard_off;   /* flat_off - owner * S */
    int64_t fill;        /* flat_off / B, or -1 without a bucket plan */
    int64_t bucket_off;  /* flat_off - fill * B, or -1 without a bucket plan */
} zero_segment;

/* Build the layout of a list of tensors flattened in list order (no
 * per-tensor padding) and cut into n_ranks equal shards of S elements.
 *   numel        host, n_tensors sizes (>= 0); may be NULL when n_tensors == 0
 *   n_ranks      N >= 1
 *   stage        0..3 (which kinds are partitioned, for the byte counts)
 *   align_elems  A >= 1: S is a multiple of A
 *   bucket_elems B >= 0: with B > 0 segments are also cut at multiples of B
 *                (the fills of the constant-size bucket)
 *   out          receives the new handle
 * Errors: INVALID_ARG (ranges), INDEX_OVERFLOW (sum of sizes, or 16 * N * S
 * bytes, beyond int64), OUT_OF_MEMORY (more than 2^26 segments). */
int zero_partition_layout(const int64_t* numel, int64_t n_tensors, int32_t n_ranks,
                          int32_t stage, int64_t align_elems, int64_t bucket_elems,
                          zero_layout** out);

int zero_layout_destroy(zero_layout* layout); /* NULL is accepted; frees device tables too */

int zero_layout_get_info(const zero_layout* layout, zero_layout_info* info);

/* Flat offset of every tensor (host, n_tensors entries).  CAPACITY when
 * cap < n_tensors. */
int zero_layout_tensor_offsets(const zero_layout* layout, int64_t* out, int64_t cap);

/* Rank r owns [begin, end); [begin, real_end) are model elements and
 * [real_end, end) padding.  INVALID_ARG unless 0 <= rank < n_ranks. */
int zero_layout_rank_range(const zero_layout* layout, int32_t rank,
                           int64_t* begin, int64_t* real_end, int64_t* end);

/* Segment queries.  *n_out always receives the number of matching segments;
 * they are written to out (host) when cap is large enough, otherwise the call
 * returns CAPACITY and writes nothing (call with cap = 0 to size the array). */
int zero_layout_segments(const zero_layout* layout, zero_segment* out, int64_t cap,
                         int64_t* n_out);
int zero_layout_rank_segments(const zero_layout* layout, int32_t rank, zero_segment* out,
                              int64_t cap, int64_t* n_out);
int zero_layout_fill_segments(const zero_layout* layout, int64_t fill, zero_segment* out,
                              int64_t cap, int64_t* n_out);

/* ------------------------------------------------------------------------ */
/* Contiguous arena for one rank's buffers (memory defragmentation paragraph)*/
/* ------------------------------------------------------------------------ */

/* Buffer kinds of one rank, in the order of zero_arena_plan.offset/bytes. */
enum {
    ZERO_ARENA_PARAM16 = 0,      /* fp16 parameters: S at stage 3, else N*S    */
    ZERO_ARENA_GRAD16 = 1,       /* fp16 gradients: S at stages 2-3, else N*S  */
    ZERO_ARENA_MASTER = 2,       /* fp32 master: S at stages 1-3, else N*S     */
    ZERO_ARENA_MOMENTUM = 3,     /* fp32 momentum, as master                   */
    ZERO_ARENA_VARIANCE = 4,     /* fp32 variance, as master                   */
    ZERO_ARENA_MASTER_ALT = 5,   /* ping-pong alternates, as master            */
    ZERO_ARENA_MOMENTUM_ALT = 6,
    ZERO_ARENA_VARIANCE_ALT = 7,
    ZERO_ARENA_BUCKET = 8,       /* fp16 constant-size bucket: B               */
    ZERO_ARENA_CONTRIB0 = 9,     /* fp16 contribution r at CONTRIB0 + r: S     */
    ZERO_ARENA_KINDS = 25
};

typedef struct zero_arena_plan {
    int64_t total_bytes;                 /* size of the one allocation        */
    int64_t align_bytes;                 /* every buffer starts on a multiple */
    int64_t offset[ZERO_ARENA_KINDS];    /* byte offset, -1 when absent        */
    int64_t bytes[ZERO_ARENA_KINDS];     /* byte size, 0 when absent           */
} zero_arena_plan;

/* Lay out one rank's buffers in a single contiguous block (host only; the
 * caller allocates total_bytes once and carves the buffers).  Element sizes
 * follow the model-states paragraph and the partitioned kinds the stage
 * paragraphs, so the five model-state kinds add up to the page's per-rank
 * bytes (plus padding).  Order: fp32 state, alternates, fp16 gradients,
 * contributions, fp16 parameters, bucket.
 *   pingpong     1: also the alternate master/momentum/variance set
 *   n_contrib    0..16 fp16 contribution buffers of S elements
 *   with_bucket  1: one bucket of B elements (the layout needs a bucket plan)
 *   align_bytes  power of two >= 256 (0: 2 MiB)
 * Errors: INVALID_ARG, STATE (bucket requested without a bucket plan),
 * INDEX_OVERFLOW. */
int zero_arena_plan_for(const zero_layout* layout, int32_t pingpong, int32_t n_contrib,
                        int32_t with_bucket, int64_t align_bytes, zero_arena_plan* out);

/* ------------------------------------------------------------------------ */
/* Bucket pack (constant-size buffers paragraph)                             */
/* ------------------------------------------------------------------------ */

/* Record the device address of every tensor of the layout and upload the
 * gather tables the pack kernel reads (on the current device, ordered on
 * `stream`; the call waits for the upload).
 *   dev_ptrs  host array of n_tensors device pointers to fp16 data, each
 *             2-byte aligned; NULL entries are allowed for zero-sized tensors.
 *             Pointer i must address at least numel[i] elements (the sizes
 *             the layout was built with): the pack reads exactly that many,
 *             and device sizes cannot be checked here.
 * The tensors must stay allocated while the layout is used for packing.
 * Binding again replaces the previous table.  Errors: STATE (layout has no
 * bucket plan), INVALID_ARG, ALIGNMENT, HIP, OUT_OF_MEMORY. */
int zero_layout_bind_tensors(zero_layout* layout, const uint16_t* const* dev_ptrs,
                             void* stream);

/* Write fill `fill` of the bucket: bucket[j] = flat[fill * B + j] for
 * fill * B + j < psi and 0x0000 past the end, where flat is the concatenation
 * of the bound tensors in list order.  A bit copy (NaN payloads, -0 kept).
 *   bucket        device, B elements, 16-byte aligned
 *   packed_elems  optional host output: min(B, psi - fill * B)
 * Asynchronous on `stream`; must run on the device the layout was bound on.
 * Errors: STATE (not bound, or another device), INVALID_ARG (fill outside
 * [0, n_fills), or B above ZERO_MAX_SHARD_ELEMS), ALIGNMENT, HIP. */
int zero_pack_bucket(const zero_layout* layout, int64_t fill, uint16_t* bucket,
                     void* stream, int64_t* packed_elems);

/* ------------------------------------------------------------------------ */
/* Bucket reduce-to-owner (Stage 2 paragraph with the constant-size buffer)  */
/* ------------------------------------------------------------------------ */

/* Record R lists of device tensors, one list per reducing rank, each with
 * the layout's tensor sizes in list order, for zero_reduce_to_owner.
 *   R         1..16
 *   dev_ptrs  host array of R * n_tensors device pointers to fp16 data; row r
 *             (entries r*n_tensors ... r*n_tensors + n_tensors - 1) holds rank
 *             r's tensors; each 2-byte aligned; NULL allowed for empty ones;
 *             each must address at least numel[i] elements, as for
 *             zero_layout_bind_tensors.
 * Uploads the tables on the current device (the call waits for the upload).
 * The tensors must stay allocated while the layout reduces.  Binding again
 * replaces the previous contribution table; the pack binding is separate.
 * Errors: STATE (no bucket plan), INVALID_ARG, ALIGNMENT, HIP, OUT_OF_MEMORY. */
int zero_layout_bind_contributions(zero_layout* layout, int32_t R,
                                   const uint16_t* const* dev_ptrs, void* stream);

/* Owner's share of the reduce of bucket fill `fill`: for every flat index g
 * with fill*B <= g < (fill+1)*B, rank*S <= g < (rank+1)*S and g < psi,
 *   shard[g - rank*S] = fp16( c_0(g) + c_1(g) + ... + c_{R-1}(g) )
 * where c_r is rank r's bound tensor list laid back to back in list order,
 * the sum is formed in fp32 from contribution 0 up and rounded once to fp16
 * (nearest, ties to even); an infinite sum is written as fp16 infinity and a
 * NaN sum as an fp16 NaN (its payload bits are not specified).  Every other
 * element of `shard` is left as it is.
 *   shard    device, the owner's fp16 gradient shard (S values), 2-byte aligned
 *   written  optional host output: elements written (0 when the fill and the
 *            rank's shard do not meet)
 * Asynchronous on `stream`; must run on the device the contributions were
 * bound on.  Errors: STATE (no bucket plan, not bound, another device),
 * INVALID_ARG (fill or rank out of range, B above ZERO_MAX_SHARD_ELEMS),
 * ALIGNMENT, HIP. */
int zero_reduce_to_owner(const zero_layout* layout, int64_t fill, int32_t rank,
                         uint16_t* shard, void* stream, int64_t* written);

/* ------------------------------------------------------------------------ */
/* Fused shard step (Stage 1/2/3 paragraphs: the rank's own partition)        */
/* ------------------------------------------------------------------------ */

/* fp32 shard state of one rank.  Set [cur] is the live state.  When
 * p[1], m[1] and v[1] are all NULL the step runs in place (two passes over
 * the gradients: an overflow check, then the update).  When all three are
 * given the step reads set [cur] and writes set [1 - cur] in one pass, and
 * a taken step flips `cur` (ping-pong mode).  All six pointers are device
 * pointers to shard_elems floats, 16-byte aligned, and the sets may not
 * overlap. */
typedef struct zero_shard_state {
    int64_t shard_elems;   /* S */
    float* p[2];           /* fp32 master parameters */
    float* m[2];           /* fp32 momentum (first moment) */
    float* v[2];           /* fp32 variance (second moment) */
    int32_t cur;           /* live set: 0 or 1 (always 0 in place) */
    int32_t reserved;
    int64_t t;             /* Adam steps taken so far (skipped steps excluded) */
} zero_shard_state;

/* All finite; beta1, beta2 in [0, 1); eps > 0 (with eps = 0 a zero gradient
 * on a zero variance would divide 0 by 0). */
typedef struct zero_adam_hparams {
    float lr;
    float beta1;
    float beta2;
    float eps;
    float weight_decay;    /* L2 term added to the gradient; 0 disables it */
} zero_adam_hparams;

/* Dynamic loss scale.  A step is skipped when any reduced gradient value is
 * inf or NaN: then scale = max(scale * backoff, min_scale), good_steps = 0
 * and no state changes.  A taken step increments good_steps (saturating at INT32_MAX), and when it
 * reaches growth_interval (> 0) the scale is multiplied by growth (kept when
 * that product is not finite) and good_steps reset.
 *
 * scale and min_scale must be at least ZERO_MIN_LOSS_SCALE (2^-24); calls
 * with a smaller value fail with ZERO_ERR_INVALID_ARG.  At or above it
 * 1/scale is finite, and a finite sum of at most 16 fp16 values (below 2^20
 * in magnitude) unscales to |g| < 2^44, whose square stays far inside the
 * fp32 range: a clean step never turns a finite gradient into inf or NaN. */
#define ZERO_MIN_LOSS_SCALE 5.9604644775390625e-08f

/* Largest shard a step call takes, and largest bucket the pack and the
 * reduce-to-owner take (4096 * (2^24 - 1) elements, about 6.9e10): a pass is
 * one launch of 256-thread workgroups of 4096 elements each, and HIP takes
 * fewer than 2^32 work-items per grid dimension, so at most 2^24 - 1 of them.
 * Larger shard_elems (or bucket_elems) fail with ZERO_ERR_INVALID_ARG. */
#define ZERO_MAX_SHARD_ELEMS 68719472640LL
typedef struct zero_loss_scaler {
    float scale;           /* the contributions were multiplied by this */
    float backoff;
    float growth;
    float min_scale;
    int32_t growth_interval;
    int32_t good_steps;
} zero_loss_scaler;

/* One rank's shard step:
 *   sum   = grads[0] + grads[1] + ... + grads[R-1]   (fp16 inputs, fp32
 *           additions in that order)
 *   flag  = any element of sum is inf or NaN (over all S elements)
 *   if flag: skip (no state change), scaler backs off
 *   else, with t = st->t + 1:
 *     g = sum * (1 / scale) [+ weight_decay * p]
 *     m = beta1 * m + (1 - beta1) * g
 *     v = beta2 * v + (1 - beta2) * g * g
 *     p = p - lr * (m / (1 - beta1^t)) / (sqrt(v / (1 - beta2^t)) + eps)
 *     out_slot = fp16(p), round to nearest even
 *     st->t = t, scaler counts a good step
 *   grads     host array of R device pointers to S fp16 values each,
 *             16-byte aligned (the R contributions to this rank's slice)
 *   R         1..16
 *   out_slot  device, S fp16 values, 2-byte aligned: this rank's slot of the
 *             gather buffer (gather + rank * S)
 *   overflow  host output: 1 if the step was skipped, else 0 (may be NULL)
 * The call returns once the overflow decision is known: the last block of
 * the pass writes it into a pinned host word that the call polls, querying
 * `stream` meanwhile (an error on the stream, or a stream that drains
 * without the word written, ends the wait with an error).  In ping-pong mode
 * the pass may still be retiring when the call returns; in place the call
 * also waits for `stream`.  Everything the call enqueues (the passes, and
 * restoring the slot of a skipped ping-pong step) is ordered on `stream`:
 * order later readers of the state or the slot after it.  Calls on one
 * device are serialised by the library.
 * Errors: INVALID_ARG, ALIGNMENT, STATE, HIP. */
int zero_shard_step(zero_shard_state* st, const uint16_t* const* grads, int32_t R,
                    const zero_adam_hparams* hp, zero_loss_scaler* scaler,
                    uint16_t* out_slot, void* stream, int32_t* overflow);

/* zero_shard_step for callers that cannot allocate memory (code that must
 * not call hipMalloc or hipHostMalloc: tight serving loops, harnesses that
 * forbid allocation).  Same arguments, arithmetic, results, errors and
 * state/scaler updates as zero_shard_step, bit for bit, on the same kernels.
 * What differs: the flag word, the blocks-done counter and the decision word
 * live in a fixed 256-byte device array of the library (one copy per device
 * and process, kept until the process ends) instead of a workspace allocated
 * on a device's first call, and the call clears those words on `stream`
 * (with a one-block kernel),
 * copies the 8-byte decision back into host memory after the pass and waits
 * for `stream` (zero_shard_step instead polls a pinned host word).  The array
 * keeps the last call's contents; calls on one device are serialised by the
 * library within a process, so they never share the words at the same time.
 * The call allocates nothing (no hipMalloc, hipHostMalloc or event) and does
 * not take part in kernel timing.  The words are the same for every shard
 * size: the largest shard is ZERO_MAX_SHARD_ELEMS, as for zero_shard_step.
 * Errors: as zero_shard_step. */
int zero_shard_step_noalloc(zero_shard_state* st, const uint16_t* const* grads, int32_t R,
                            const zero_adam_hparams* hp, zero_loss_scaler* scaler,
                            uint16_t* out_slot, void* stream, int32_t* overflow);

/* Owner step: zero_shard_step in ping-pong mode with the sum taken straight
 * from the contribution lists bound by zero_layout_bind_contributions, so the
 * Stage 2 reduce of the rank's partition and its Stage 1 update are one pass
 * and no fp16 gradient shard is written in between.  With n = the rank's real
 * elements (min(S, psi - rank*S), or 0),
 *   sum(j) = c_0(rank*S + j) + ... + c_{R-1}(rank*S + j)   for j < n
 *   sum(j) = 0                                             for n <= j < S
 * (fp16 values, fp32 additions from contribution 0 up; c_r as for
 * zero_reduce_to_owner; no gradient reaches the padding), the flag, the Adam
 * arithmetic, the slot, the skip and the loss-scale rule are those of
 * zero_shard_step over all S elements: the result equals zero_shard_step fed
 * with the rank's windows of the R flattened lists, zero-filled past the end
 * of the model.  Padding that starts at 0 therefore stays 0 in the live set
 * and the slot, whatever the alternate set held.
 *   layout    bucket plan with contributions bound on the current device
 *   rank      0 .. n_ranks - 1: whose partition is updated
 *   st        ping-pong state (p[1], m[1], v[1] set), shard_elems = the
 *             layout's S; 16-byte aligned, pairwise disjoint, disjoint from
 *             every bound contribution tensor
 *   out_slot  device, S fp16 values, 2-byte aligned (gather + rank * S)
 *   overflow  host output: 1 if the step was skipped, else 0 (may be NULL)
 * Returns once the overflow decision is known (a one-thread kernel after the
 * pass writes it into the pinned host word the call polls, as for
 * zero_shard_step); the pass, and restoring the slot of a skipped step, are
 * ordered on `stream`.  Calls on one device are serialised by the library,
 * together with zero_shard_step.
 * Errors: INVALID_ARG (rank, in-place state, S mismatch, overlap),
 * ALIGNMENT, STATE (no bucket plan, not bound, another device), HIP. */
int zero_owner_step(const zero_layout* layout, int32_t rank, zero_shard_state* st,
                    const zero_adam_hparams* hp, zero_loss_scaler* scaler,
                    uint16_t* out_slot, void* stream, int32_t* overflow);

/* ------------------------------------------------------------------------ */
/* Kernel timing (profiling aid)                                            */
/* ------------------------------------------------------------------------ */

/* Per calling thread.  While enabled (enable != 0), zero_shard_step,
 * zero_owner_step, zero_pack_bucket and zero_reduce_to_owner time their
 * kernels with a pair of HIP events that the launch itself records at the
 * start of their first kernel and at the end of their last (for
 * zero_shard_step: the fused pass, or the check and update passes in place;
 * for zero_owner_step: the pass, without the one-thread flag hand-over).
 * The pairs go into a ring of 4096 per thread, so calls can be timed back to
 * back without waiting on the events; enabling or disabling clears it.
 * zero_last_kernel_ms waits for the most recent pair's end event and returns
 * its elapsed milliseconds.  Errors: STATE (nothing recorded since enabling),
 * HIP. */
int zero_set_kernel_timing(int32_t enable);
int zero_last_kernel_ms(float* ms);

/* The elapsed milliseconds of every call timed since timing was enabled
 * (at most the last 4096), oldest first, into ms[0 .. *n); waits for their
 * events.  *n is always set; ms may be NULL when *n is 0.
 * Errors: INVALID_ARG (n NULL), CAPACITY (cap < *n), HIP. */
int zero_kernel_times(float* ms, int64_t cap, int64_t* n);

/* ------------------------------------------------------------------------ */
/* Misc                                                                      */
/* ------------------------------------------------------------------------ */

int zero_version(void);
const char* zero_last_error(void);     /* thread-local, never NULL */
int zero_last_hip_error(void);         /* hipError_t of the last ZERO_ERR_HIP */

/* sizeof of the ABI structs, for binding checks: 0 layout_info, 1 segment,
 * 2 shard_state, 3 adam_hparams, 4 loss_scaler, 5 arena_plan; -1 otherwise. */
int64_t zero_abi_struct_size(int32_t which);

/* Architecture of the current device as a number (gfx950 -> 950) and its
 * memory size in bytes. */
int zero_device_info(int32_t* arch, int64_t* hbm_bytes);

#ifdef __cplusplus
}
#endif

#endif /* ZERO_PARTITION_H */
