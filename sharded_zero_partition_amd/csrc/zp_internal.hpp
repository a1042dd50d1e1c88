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

struct ReduceLaunch {
    const int64_t* off;          // device, n_src flat offsets (sorted)
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
};

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

}  // namespace zp
