// zp_internal.hpp -- declarations shared by the library's host and device
// translation units (not part of the public ABI).
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>
#include <string>
#include <vector>

#include "zero_partition.h"

namespace zp {

// ---------------------------------------------------------------------------
// error reporting (thread-local message, see capi.cpp)
// ---------------------------------------------------------------------------
int fail(int status, const std::string& msg);
int fail_hip(hipError_t err, const char* what);

// The events of one timed call (both null when timing is off).
struct KernelEvents {
    hipEvent_t start = nullptr;
    hipEvent_t stop = nullptr;
};
void clear_error();

// ---------------------------------------------------------------------------
// work order of the span kernels (pack, reduce-to-owner, owner step)
// ---------------------------------------------------------------------------

// A wave of these kernels owns a span of kSpanElems consecutive elements
// (kSpanVecs vectors of 8); span w starts at flat index span0 + kSpanElems w.
// A span inside one tensor takes a cooperative path (one aligned load per
// lane and contribution, the misalignment fixed up by cross-lane shuffles);
// a span near a tensor boundary takes a slower one.  So that the slow spans
// do not end up among the last waves of a launch, where their longer
// latency would hold up the launch's end, the first n_hard waves take them:
//   wave 0 and wave 1: spans 0 and n_span - 1 (the ends of the range);
//   wave 2 + hard_per_b q + j: the j-th span "claimed" by boundary b_first + q.
// The boundaries are the flat offsets of the tensors, then psi (the end of
// the last tensor).  Boundary b claims the interior span w
// (1 <= w <= n_span - 2) when
//     cs(F(w) - 7) < b < F(w + 1) + 8,
// F(w) being the span's first flat index and cs(x) the start of the chunk
// (of the tables' chunk index) holding x; a span claimed by several
// boundaries belongs to the lowest.  A boundary claims at most
// chunk / kSpanElems + 2 spans, the value of hard_per_b.
// Wave n_hard + w takes the interior span w when no boundary claims it.  It
// reads the tensor t holding the start of the chunk that holds F(w) - 7: t's
// end is the first boundary after that chunk start, so no boundary claims
// the span exactly when t ends at or after F(w + 1) + 8, and then t holds
// the span, the 7 elements before it and the 8 after it.
// When the boundary waves would far outnumber the spans (many tiny tensors
// in a short range), or the grid would pass the launch limit, the launch
// runs in order instead (hard_per_b = 0, n_hard = 0): wave w takes span w,
// whatever it holds.
constexpr int64_t kSpanVecs = 128;
constexpr int64_t kSpanElems = 8 * kSpanVecs;
constexpr int kSpanShift = 10;
static_assert(int64_t(1) << kSpanShift == kSpanElems, "span length");

// Waves of one launch of 256-thread workgroups: HIP takes fewer than 2^32
// work-items per grid dimension.
constexpr int64_t kMaxGridWaves = ((int64_t(1) << 24) - 1) * 4;

struct HardWaves {
    int64_t n_hard;      // waves ahead of the span waves
    int64_t b_first;     // first boundary (index into the offsets) that claims a span
    int32_t hard_per_b;  // waves per boundary; 0: in order (no hard waves)
};

// The plan for n_span spans from flat index span0, with off the host copy of
// the boundaries (n_off ascending flat offsets, the last psi) and
// chunk_shift that of the tables.  Pure host arithmetic.
HardWaves plan_hard_waves(const int64_t* off, int64_t n_off, int chunk_shift, int64_t span0, int64_t n_span);

// The span hard wave `wave` (< n_hard) takes, or -1.  off(i) is boundary i.
template <class Off>
__host__ __device__ inline int64_t hard_wave_span(int64_t wave, int64_t n_span, int64_t span0, const HardWaves& h,
                                                  int chunk_shift, const Off& off) {
    if (wave < 2) {   // the ends of the range
        if (wave == 1 && n_span == 1) return -1;
        return wave == 0 ? 0 : n_span - 1;
    }
    // the j-th span claimed by boundary i, less those the previous boundary
    // claims (the boundaries claiming one span are consecutive)
    const int64_t q = (wave - 2) / h.hard_per_b;
    const int64_t j = (wave - 2) - q * h.hard_per_b;
    const int64_t i = h.b_first + q;
    const int s = chunk_shift;
    const int64_t b = off(i);
    const int64_t nc = (((b - 1) >> s) + 1) << s;            // cs(x) < b exactly when x < nc
    int64_t w_lo = (b - 8 - span0) >> kSpanShift;            // F(w + 1) + 8 > b
    int64_t w_hi = (nc + 6 - span0) >> kSpanShift;           // F(w) - 7 < nc
    if (i > h.b_first) {
        const int64_t bp = off(i - 1);
        const int64_t ncp = (((bp - 1) >> s) + 1) << s;
        // the previous boundary claims w while F(w) - 7 < ncp
        const int64_t w_new = (ncp + 7 - span0 + kSpanElems - 1) >> kSpanShift;
        if (w_new > w_lo) w_lo = w_new;
    }
    if (w_lo < 1) w_lo = 1;
    if (w_hi > n_span - 2) w_hi = n_span - 2;
    const int64_t w = w_lo + j;
    return w > w_hi ? -1 : w;
}

// Whether a boundary claims the interior span starting at flat index f,
// from the tensor holding the start of the chunk that holds f - 7 (its flat
// offset and length).
__host__ __device__ inline bool span_claimed(int64_t t_off, int64_t t_len, int64_t f) {
    return t_off + t_len < f + kSpanElems + 8;
}

// ---------------------------------------------------------------------------
// pack kernel tables
// ---------------------------------------------------------------------------

// One non-empty tensor of the flattened stream, as the pack kernel sees it.
struct PackSrc {
    const uint16_t* ptr;  // device address of element 0
    int64_t flat_off;     // first flat index
    int64_t len;          // elements (> 0)
};

struct PackLaunch {
    const PackSrc* src;       // device, n_src entries sorted by flat_off
    const int32_t* first;     // device, n_chunks + 1 entries: src index holding
                              // flat index c << chunk_shift (last entry n_src - 1)
    int32_t n_src;
    int32_t chunk_shift;
    int64_t psi;
    int64_t fill_base;        // fill * B
    int64_t bucket_elems;     // B
    uint16_t* bucket;         // device, 16-byte aligned
    int64_t n_span;           // spans of the fill: ceil(B / kSpanElems)
    int64_t n_data_span;      // spans holding elements below psi (the rest are zeros)
    HardWaves hard;           // the work order over spans [0, n_data_span)
};

hipError_t launch_pack(const PackLaunch& a, hipStream_t stream, const KernelEvents& ev);

// ---------------------------------------------------------------------------
// bucket reduce-to-owner
// ---------------------------------------------------------------------------

constexpr int kMaxReduceRanks = 16;

// Bytes of one per-chunk record of the reduce tables for R contributions:
// int64 flat offset (byte 0), int64 length (8), int32 tensor index (16), 4
// bytes padding, then R device addresses (24 + 8 r); rounded up to 16.
constexpr int chunk_rec_bytes(int R) { return (24 + 8 * R + 15) / 16 * 16; }

// The reduce-to-owner and owner-step kernels cut the owner's shard into
// 8-element vectors on its own 16-byte grid (vector k covers shard
// positions [8k - mis, 8k - mis + 8), mis = the shard's misalignment in
// elements); span 0 starts at the vector holding the range's first position.
struct SpanGeometry {
    int64_t k_lo;     // first vector
    int64_t k_end;    // one past the last vector
    int64_t n_span;   // spans
    int64_t span0;    // flat index of span 0's first position (may precede the range)
};

// Span grid over shard positions [j_lo, j_hi) (j_hi > j_lo) of the shard
// starting at flat index base.
__host__ __device__ inline SpanGeometry span_geometry(int64_t base, int64_t j_lo, int64_t j_hi, int mis) {
    SpanGeometry g;
    g.k_lo = (j_lo + mis) >> 3;
    g.k_end = ((j_hi - 1 + mis) >> 3) + 1;
    g.n_span = (g.k_end - g.k_lo + kSpanVecs - 1) / kSpanVecs;
    g.span0 = base + 8 * g.k_lo - mis;
    return g;
}

struct ReduceLaunch {
    const int64_t* off;          // device, n_src + 1 flat offsets (sorted; off[n_src] = psi)
    const int64_t* len;          // device, n_src lengths (> 0)
    const uint16_t* const* ptr;  // device, R * n_src addresses, row r = rank r
    const int32_t* first;        // device chunk index, as in PackLaunch
    const uint8_t* rec;          // device, one chunk_rec_bytes(R) record per chunk c:
                                 // the entries of tensor first[c]
    int32_t n_src;
    int32_t chunk_shift;
    int32_t R;
    int64_t g_lo;                // reduce flat indices [g_lo, g_hi)
    int64_t g_hi;
    int64_t base;                // flat index of shard[0] (rank * S)
    uint16_t* shard;             // device, 2-byte aligned
    int64_t n_span;              // spans of the range (span_geometry)
    HardWaves hard;              // the work order (plan_hard_waves over the offsets)
};

// Fills n_span and hard of `a` (whose range and base are set) for a shard
// misaligned by `mis` elements; off, n_off and chunk_shift as for
// plan_hard_waves.
void plan_reduce_waves(const int64_t* off, int64_t n_off, int chunk_shift, int mis, ReduceLaunch* a);

hipError_t launch_reduce_owner(const ReduceLaunch& a, hipStream_t stream, const KernelEvents& ev);

// ---------------------------------------------------------------------------
// shard step kernels
// ---------------------------------------------------------------------------

constexpr int kMaxContrib = 16;

struct StepLaunch {
    const uint16_t* grad[kMaxContrib];  // R device pointers, 16-byte aligned
    int32_t R;
    const float* p_in;
    const float* m_in;
    const float* v_in;
    float* p_out;       // == p_in in place
    float* m_out;
    float* v_out;
    uint16_t* out16;    // fp16 slot, 2-byte aligned
    int64_t n;          // S
    float inv_scale;    // 1 / scale
    float lr;
    float beta1;
    float beta2;
    float one_minus_beta1;
    float one_minus_beta2;
    float bias_corr1;   // 1 - beta1^t
    float bias_corr2;   // 1 - beta2^t
    float eps;
    float weight_decay;
    uint32_t* flag;     // device word; set to `epoch` when a value is not finite
    uint32_t epoch;
    unsigned long long* done;        // device word, 0 between launches: blocks finished
                                     // (high 32 bits) and blocks that saw a non-finite
                                     // value (low 32 bits) in the current pass
    unsigned long long* host_word;   // pinned host word: (epoch << 1) | flag, written by
                                     // the last block of a flag-raising pass
};

// One pass: reduce + finite check + Adam + fp16 cast, reading set *_in and
// writing set *_out (distinct buffers); raises the flag and publishes it to
// the host word.
hipError_t launch_fused_step(const StepLaunch& a, hipStream_t stream, const KernelEvents& ev);

// In-place mode, pass 1: finite check over the R contributions only; raises
// the flag and publishes it to the host word.
hipError_t launch_check(const StepLaunch& a, int cu_count, hipStream_t stream, hipEvent_t start);

// In-place mode, pass 2: the update, skipped by every thread when the flag
// already holds `epoch`.
hipError_t launch_update_in_place(const StepLaunch& a, hipStream_t stream, hipEvent_t stop);

// Rewrite the fp16 slot from the fp32 master values (restores the slot after
// a skipped ping-pong step): out16[i] = fp16(p_in[i]).
hipError_t launch_slot_from_master(const StepLaunch& a, int cu_count, hipStream_t stream);

// ---------------------------------------------------------------------------
// owner step: the shard step fed straight from the R ranks' ragged tensors
// ---------------------------------------------------------------------------

// The reduce-to-owner tables and range (the `shard` member unused) plus the
// shard step's state pointers and constants (its `grad` members unused).
// Element j of the owner's shard is flat index base + j; the range
// [g_lo, g_hi) is the owner's real elements.  p/m/v 16-byte aligned.
struct OwnerLaunch : ReduceLaunch {
    StepLaunch st;
};

// One pass over the range: reduce, Adam (reading set *_in, writing *_out) and
// the fp16 slot; a wave that saw a non-finite sum raises st.flag to st.epoch.
// A one-thread kernel after it writes (epoch << 1) | flag to st.host_word.
hipError_t launch_owner_step(const OwnerLaunch& a, hipStream_t stream, const KernelEvents& ev);

// The reduce tables bound on `l` (layout.cpp) for an owner step of `rank`:
// fills every ReduceLaunch member but `shard`, with [g_lo, g_hi) the rank's
// real elements (empty when its shard is all padding), and the device the
// tables live on.  Makes no HIP call.
int owner_tables(const zero_layout* l, int32_t rank, ReduceLaunch* out, int* bound_dev);

// True when the byte range [lo, hi) meets a bound contribution tensor of `l`.
bool contributions_overlap(const zero_layout* l, uintptr_t lo, uintptr_t hi);

// ZERO_OK when `stream` (NULL = the null stream) belongs to device `dev`,
// else a STATE error naming `what`.
int check_stream_device(void* stream, int dev, const char* what);

// Kernel timing (zero_set_kernel_timing): begin/end mark the first and last
// kernel of a call on its stream; both are no-ops while timing is disabled.
// Kernel timing: while enabled on the calling thread, timing_events hands out
// the next event pair of the thread's ring (null events otherwise), the
// launch functions attach its start to their first kernel and its stop to
// their last (hipExtLaunchKernel records the kernels' own start and end),
// and timing_done closes the pair once the launches are enqueued.
hipError_t timing_events(KernelEvents* ev);
void timing_done();

// Blocks per CU of the grid-stride kernels (the in-place check pass and the
// slot restore), read once from ZERO_BLOCKS_PER_CU when set.
int blocks_per_cu_step();

// The fixed scratch of zero_shard_step_noalloc (noalloc.hip): 64 words, 256
// bytes, one copy per device.  static_scratch returns device `dev`'s address
// of it (looked up once per device, with `dev` the current device).
constexpr int kStaticScratchWords = 64;
int static_scratch(int dev, uint32_t** out);
// Zeroes the kStaticScratchWords words at w on `stream` with a one-block kernel.
hipError_t clear_scratch(uint32_t* w, hipStream_t stream);

}  // namespace zp
