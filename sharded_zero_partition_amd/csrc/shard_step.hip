// shard_step.hip -- fused ZeRO-DP shard step for gfx950.
//
// One rank's share of the optimizer step, per the ZeRO explainer page
// ("ZeRO: Memory Optimizations Toward Training Trillion Parameter Models",
// azimuth.plus):
//   - Stage 2 (P_os+g) paragraph: the rank ends up with only its slice of the
//     reduced gradients; locally that is the sum of R fp16 contributions;
//   - Stage 1 (P_os) paragraph: the rank updates only its partition of the
//     parameters with its partition of the fp32 Adam state (model-states
//     paragraph: master copy, momentum, variance), and the new fp16
//     parameters go to its slot of the gather buffer for the all-gather.
// Adam is the textbook bias-corrected form (the page names Adam but does not
// write it out); a step with any inf/NaN in the reduced gradients is skipped
// (dynamic loss scaling; not on the page).
//
// Every element is independent and the kernel moves 26 + 2R bytes per element
// for about 80 ALU operations, so it is bound by HBM bandwidth.  Design:
//   - one 1024-element tile per wave over a full grid, so the hardware keeps
//     many short waves in flight and hands each free slot the next tile;
//     fully coalesced 128/64-bit accesses; a scalar tail for the elements
//     past the last whole tile;
//   - the fp32 arithmetic is written in the order of the definition with one
//     rounding per operation (no contraction, IEEE division and square root),
//     so the results match a scalar reference bit for bit; this costs no time
//     (the ALU work hides under the HBM traffic);
//   - the overflow flag is a block-level OR followed by one counting atomic
//     per block; the last block to finish writes the decision into a pinned
//     host word, and on overflow into the device flag word, which holds the
//     epoch of the call that raised it, so it never has to be cleared;
//   - ping-pong state (read set A, write set B) makes the step a single pass:
//     the commit is the host flipping the live set once the flag is known.
#include <hip/hip_ext.h>

#include "adam.hpp"
#include "vec16.hpp"
#include "zp_internal.hpp"

#pragma clang fp contract(off)

namespace zp {
namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

constexpr int kThreads = 256;

// fp16 slot alignment classes
constexpr int kOut16B = 0;
constexpr int kOut8B = 1;
constexpr int kOut4B = 2;
constexpr int kOut2B = 3;

template <typename T>
__device__ __forceinline__ T load_stream(const T* p) {
    return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void store_stream(T* p, T v) {
    __builtin_nontemporal_store(v, p);
}

// Sum of the R contributions of element e, contribution 0 first.
template <int R>
__device__ __forceinline__ float reduce1(const StepLaunch& a, int64_t e) {
    float s = h2f(a.grad[0][e]);
#pragma unroll
    for (int r = 1; r < R; ++r) s = s + h2f(a.grad[r][e]);
    return s;
}

template <int OUT>
__device__ __forceinline__ void store_half8(uint16_t* dst, const float p[8]) {
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = f2h(p[2 * d]) | (f2h(p[2 * d + 1]) << 16);
    if (OUT == kOut16B) {
        store_stream(reinterpret_cast<u32x4*>(dst), u32x4{w[0], w[1], w[2], w[3]});
    } else if (OUT == kOut8B) {
        store_stream(reinterpret_cast<u32x2*>(dst), u32x2{w[0], w[1]});
        store_stream(reinterpret_cast<u32x2*>(dst + 4), u32x2{w[2], w[3]});
    } else if (OUT == kOut4B) {
#pragma unroll
        for (int d = 0; d < 4; ++d) store_stream(reinterpret_cast<uint32_t*>(dst + 2 * d), w[d]);
    } else {
#pragma unroll
        for (int k = 0; k < 8; ++k) dst[k] = uint16_t(w[k >> 1] >> (16 * (k & 1)));
    }
}

// End of a flag-raising pass; every thread of every block calls it.  Each
// block ORs its threads' flags and adds (1 << 32) | block_flag to the 64-bit
// counter word with one relaxed atomic (a single location, so the counts
// cannot be reordered).  The block that completes the count knows the
// result: it sets the device flag word to `epoch` on overflow (the in-place
// update pass reads it), rearms the counter for the next launch and writes
// (epoch << 1) | flag into the pinned host word, so the host learns the
// decision without a copy or a stream synchronisation.
__device__ __forceinline__ void finish_pass(const StepLaunch& a, bool bad) {
    const int block_bad = __syncthreads_or(bad ? 1 : 0);
    if (threadIdx.x != 0) return;
    const unsigned long long mine = (1ull << 32) | (block_bad ? 1ull : 0ull);
    const unsigned long long before =
        __hip_atomic_fetch_add(a.done, mine, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    if ((before >> 32) != gridDim.x - 1) return;
    const bool flag = ((before & 0xFFFFFFFFull) != 0) || block_bad;
    if (flag) atomicMax(a.flag, a.epoch);
    __hip_atomic_store(a.done, 0ull, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long word = (static_cast<unsigned long long>(a.epoch) << 1) | (flag ? 1ull : 0ull);
    __hip_atomic_store(a.host_word, word, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// ---------------------------------------------------------------------------
// The step kernel (every R from 1 to 16).
//
// Each wave owns one tile of 1024 elements (four 256-element groups), tile t
// covering [1024 t, 1024 (t+1)), and the grid holds one wave per tile.  Lane
// l holds elements 4l..4l+3 of each group, so every load and store
// instruction of the wave touches one contiguous 1 KiB (fp32) or 512 B (fp16)
// range.  A wave loads its tile, computes, stores and ends (at R = 2 the
// compiler issues the contributions and the first two groups' p, m, v, and
// the last two groups' after the first groups' arithmetic, which keeps the
// kernel at 77 VGPRs; forcing every load first took 88 VGPRs and ran 1%
// slower); the hardware keeps several such waves per SIMD in flight (148
// VGPRs at R = 16) and hands each free slot the next tile.  On the same
// buffers this ran 3-6% faster for every R than a persistent grid (one block
// per CU) whose waves walked their tiles with a register double buffer, with
// the same results bit for bit; 512- and 2048-element tiles ran slower.
// ---------------------------------------------------------------------------

constexpr int kTileGroups = 4;                  // 256-element groups per tile
constexpr int64_t kTile = 256 * kTileGroups;    // elements per tile (one wave)

template <int R, int H>
struct TileRegs {
    u32x2 g[R][H];   // 4 fp16 values per group, per contribution
    f32x4 p[H], m[H], v[H];
};

template <int R, int H>
__device__ __forceinline__ void load_tile(const StepLaunch& a, int64_t base, int lane,
                                          TileRegs<R, H>& t) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
        const int64_t e = base + h * 256 + 4 * lane;
#pragma unroll
        for (int r = 0; r < R; ++r)
            t.g[r][h] = load_stream(reinterpret_cast<const u32x2*>(a.grad[r] + e));
        t.p[h] = load_stream(reinterpret_cast<const f32x4*>(a.p_in + e));
        t.m[h] = load_stream(reinterpret_cast<const f32x4*>(a.m_in + e));
        t.v[h] = load_stream(reinterpret_cast<const f32x4*>(a.v_in + e));
    }
}

template <int OUT>
__device__ __forceinline__ void store_half4(uint16_t* dst, const float p[4]) {
    const uint32_t w0 = f2h(p[0]) | (f2h(p[1]) << 16);
    const uint32_t w1 = f2h(p[2]) | (f2h(p[3]) << 16);
    if (OUT == kOut16B || OUT == kOut8B) {
        store_stream(reinterpret_cast<u32x2*>(dst), u32x2{w0, w1});
    } else if (OUT == kOut4B) {
        store_stream(reinterpret_cast<uint32_t*>(dst), w0);
        store_stream(reinterpret_cast<uint32_t*>(dst + 2), w1);
    } else {
        dst[0] = uint16_t(w0);
        dst[1] = uint16_t(w0 >> 16);
        dst[2] = uint16_t(w1);
        dst[3] = uint16_t(w1 >> 16);
    }
}

template <int R, int H, int OUT, bool kFlag>
__device__ __forceinline__ void compute_tile(const StepLaunch& a, int64_t base, int lane,
                                             const TileRegs<R, H>& t, bool& bad) {
#pragma unroll
    for (int h = 0; h < H; ++h) {
        const int64_t e = base + h * 256 + 4 * lane;
        float s[4];
        const uint32_t w0[2] = {t.g[0][h].x, t.g[0][h].y};
#pragma unroll
        for (int k = 0; k < 4; ++k) s[k] = h2f(w0[k >> 1] >> (16 * (k & 1)));
#pragma unroll
        for (int r = 1; r < R; ++r) {
            const uint32_t w[2] = {t.g[r][h].x, t.g[r][h].y};
#pragma unroll
            for (int k = 0; k < 4; ++k) s[k] = s[k] + h2f(w[k >> 1] >> (16 * (k & 1)));
        }
        float p[4] = {t.p[h].x, t.p[h].y, t.p[h].z, t.p[h].w};
        float m[4] = {t.m[h].x, t.m[h].y, t.m[h].z, t.m[h].w};
        float v[4] = {t.v[h].x, t.v[h].y, t.v[h].z, t.v[h].w};
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            if (kFlag) bad |= not_finite(s[k]);
            adam_element(a, s[k], p[k], m[k], v[k]);
        }
        store_stream(reinterpret_cast<f32x4*>(a.p_out + e), f32x4{p[0], p[1], p[2], p[3]});
        store_stream(reinterpret_cast<f32x4*>(a.m_out + e), f32x4{m[0], m[1], m[2], m[3]});
        store_stream(reinterpret_cast<f32x4*>(a.v_out + e), f32x4{v[0], v[1], v[2], v[3]});
        store_half4<OUT>(a.out16 + e, p);
    }
}

// kFlag: compute the overflow flag and hand it over (the fused pass).
// kSkip: in place, after the check pass -- do nothing if the flag holds this
// call's epoch.
template <int R, int OUT, bool kFlag, bool kSkip>
__global__ __launch_bounds__(kThreads) void step_tile_kernel(const StepLaunch a) {
    if (kSkip && __atomic_load_n(a.flag, __ATOMIC_RELAXED) == a.epoch) return;
    const int lane = threadIdx.x & 63;
    const int64_t ntiles = a.n / kTile;
    const int64_t t = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
    bool bad = false;
    if (t < ntiles) {
        TileRegs<R, kTileGroups> regs;
        load_tile<R, kTileGroups>(a, t * kTile, lane, regs);
        compute_tile<R, kTileGroups, OUT, kFlag>(a, t * kTile, lane, regs, bad);
    }
    // the last S mod 1024 elements: block 0, one element per thread per pass
    if (blockIdx.x == 0) {
        for (int64_t e = ntiles * kTile + threadIdx.x; e < a.n; e += kThreads) {
            const float s = reduce1<R>(a, e);
            if (kFlag) bad |= not_finite(s);
            float p = a.p_in[e], m = a.m_in[e], v = a.v_in[e];
            adam_element(a, s, p, m, v);
            a.p_out[e] = p;
            a.m_out[e] = m;
            a.v_out[e] = v;
            a.out16[e] = uint16_t(f2h(p));
        }
    }
    if (kFlag) finish_pass(a, bad);
}

// In-place pass 1: overflow check over the contributions alone.  A sum of at
// most 16 finite fp16 values is finite in fp32 (16 * 65504 << FLT_MAX), and
// inf or NaN in any input makes the fp32 sum inf or NaN, so "some sum is not
// finite" is "some input has the all-ones fp16 exponent".
__device__ __forceinline__ bool half_special(uint32_t w) {
    return ((w & 0x7C00u) == 0x7C00u) || ((w & 0x7C000000u) == 0x7C000000u);
}

template <int R>
__global__ __launch_bounds__(kThreads) void check_kernel(const StepLaunch a) {
    const int64_t nvec = a.n >> 3;
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    const int64_t tid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    bool bad = false;
    constexpr int kMax = R == 0 ? kMaxContrib : R;
    for (int64_t i = tid; i < nvec; i += stride) {
#pragma unroll
        for (int r = 0; r < kMax; ++r) {
            if (R == 0 && r >= a.R) break;
            const u32x4 c = load_stream(reinterpret_cast<const u32x4*>(a.grad[r] + (i << 3)));
            bad = bad || half_special(c.x) || half_special(c.y) || half_special(c.z) || half_special(c.w);
        }
    }
    const int64_t tail = a.n - (nvec << 3);
    if (tid < tail) {
        const int64_t e = (nvec << 3) + tid;
#pragma unroll
        for (int r = 0; r < kMax; ++r) {
            if (R == 0 && r >= a.R) break;
            bad |= (a.grad[r][e] & 0x7C00u) == 0x7C00u;
        }
    }
    finish_pass(a, bad);
}

template <int OUT>
__global__ __launch_bounds__(kThreads) void slot_kernel(const StepLaunch a) {
    const int64_t nvec = a.n >> 3;
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    const int64_t tid = int64_t(blockIdx.x) * kThreads + threadIdx.x;
    for (int64_t i = tid; i < nvec; i += stride) {
        const int64_t e0 = i << 3;
        const f32x4 p0 = load_stream(reinterpret_cast<const f32x4*>(a.p_in + e0));
        const f32x4 p1 = load_stream(reinterpret_cast<const f32x4*>(a.p_in + e0 + 4));
        const float p[8] = {p0.x, p0.y, p0.z, p0.w, p1.x, p1.y, p1.z, p1.w};
        store_half8<OUT>(a.out16 + e0, p);
    }
    const int64_t tail = a.n - (nvec << 3);
    if (tid < tail) {
        const int64_t e = (nvec << 3) + tid;
        a.out16[e] = uint16_t(f2h(a.p_in[e]));
    }
}

int out_class(const uint16_t* p) {
    const uintptr_t x = reinterpret_cast<uintptr_t>(p);
    if ((x & 15) == 0) return kOut16B;
    if ((x & 7) == 0) return kOut8B;
    if ((x & 3) == 0) return kOut4B;
    return kOut2B;
}

dim3 grid_for(int64_t n, int cu_count, int per_cu) {
    const int64_t nvec = n >> 3;
    int64_t blocks = (nvec + kThreads - 1) / kThreads;
    const int64_t cap = int64_t(cu_count > 0 ? cu_count : 256) * per_cu;
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;   // the tail needs one block even when nvec == 0
    return dim3(unsigned(blocks));
}

template <bool kFlag, bool kSkip, int R>
void launch_tiles_r(const StepLaunch& a, hipStream_t s, const KernelEvents& ev) {
    constexpr int64_t kWavesPerBlock = kThreads / 64;
    const int64_t ntiles = a.n / kTile;
    int64_t blocks = (ntiles + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks < 1) blocks = 1;   // block 0 also owns the tail
    const dim3 grid{unsigned(blocks)};
    switch (out_class(a.out16)) {
        case kOut16B: hipExtLaunchKernelGGL((step_tile_kernel<R, kOut16B, kFlag, kSkip>), grid, dim3(kThreads), 0, s, ev.start, ev.stop, 0, a); break;
        case kOut8B: hipExtLaunchKernelGGL((step_tile_kernel<R, kOut8B, kFlag, kSkip>), grid, dim3(kThreads), 0, s, ev.start, ev.stop, 0, a); break;
        case kOut4B: hipExtLaunchKernelGGL((step_tile_kernel<R, kOut4B, kFlag, kSkip>), grid, dim3(kThreads), 0, s, ev.start, ev.stop, 0, a); break;
        default: hipExtLaunchKernelGGL((step_tile_kernel<R, kOut2B, kFlag, kSkip>), grid, dim3(kThreads), 0, s, ev.start, ev.stop, 0, a); break;
    }
}

template <bool kFlag, bool kSkip>
void launch_step(const StepLaunch& a, hipStream_t s, const KernelEvents& ev) {
    switch (a.R) {
        case 1: launch_tiles_r<kFlag, kSkip, 1>(a, s, ev); break;
        case 2: launch_tiles_r<kFlag, kSkip, 2>(a, s, ev); break;
        case 3: launch_tiles_r<kFlag, kSkip, 3>(a, s, ev); break;
        case 4: launch_tiles_r<kFlag, kSkip, 4>(a, s, ev); break;
        case 5: launch_tiles_r<kFlag, kSkip, 5>(a, s, ev); break;
        case 6: launch_tiles_r<kFlag, kSkip, 6>(a, s, ev); break;
        case 7: launch_tiles_r<kFlag, kSkip, 7>(a, s, ev); break;
        case 8: launch_tiles_r<kFlag, kSkip, 8>(a, s, ev); break;
        case 9: launch_tiles_r<kFlag, kSkip, 9>(a, s, ev); break;
        case 10: launch_tiles_r<kFlag, kSkip, 10>(a, s, ev); break;
        case 11: launch_tiles_r<kFlag, kSkip, 11>(a, s, ev); break;
        case 12: launch_tiles_r<kFlag, kSkip, 12>(a, s, ev); break;
        case 13: launch_tiles_r<kFlag, kSkip, 13>(a, s, ev); break;
        case 14: launch_tiles_r<kFlag, kSkip, 14>(a, s, ev); break;
        case 15: launch_tiles_r<kFlag, kSkip, 15>(a, s, ev); break;
        default: launch_tiles_r<kFlag, kSkip, 16>(a, s, ev); break;
    }
}

}  // namespace

hipError_t launch_fused_step(const StepLaunch& a, hipStream_t stream, const KernelEvents& ev) {
    launch_step<true, false>(a, stream, ev);
    return hipGetLastError();
}

hipError_t launch_update_in_place(const StepLaunch& a, hipStream_t stream, hipEvent_t stop) {
    KernelEvents ev;
    ev.stop = stop;
    launch_step<false, true>(a, stream, ev);
    return hipGetLastError();
}

hipError_t launch_check(const StepLaunch& a, int cu_count, hipStream_t stream, hipEvent_t start) {
    const dim3 grid = grid_for(a.n, cu_count, blocks_per_cu_step());
    switch (a.R) {
        case 1: hipExtLaunchKernelGGL(check_kernel<1>, grid, dim3(kThreads), 0, stream, start, nullptr, 0, a); break;
        case 2: hipExtLaunchKernelGGL(check_kernel<2>, grid, dim3(kThreads), 0, stream, start, nullptr, 0, a); break;
        case 4: hipExtLaunchKernelGGL(check_kernel<4>, grid, dim3(kThreads), 0, stream, start, nullptr, 0, a); break;
        default: hipExtLaunchKernelGGL(check_kernel<0>, grid, dim3(kThreads), 0, stream, start, nullptr, 0, a); break;
    }
    return hipGetLastError();
}

hipError_t launch_slot_from_master(const StepLaunch& a, int cu_count, hipStream_t stream) {
    const dim3 grid = grid_for(a.n, cu_count, blocks_per_cu_step());
    switch (out_class(a.out16)) {
        case kOut16B: hipLaunchKernelGGL(slot_kernel<kOut16B>, grid, dim3(kThreads), 0, stream, a); break;
        case kOut8B: hipLaunchKernelGGL(slot_kernel<kOut8B>, grid, dim3(kThreads), 0, stream, a); break;
        case kOut4B: hipLaunchKernelGGL(slot_kernel<kOut4B>, grid, dim3(kThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL(slot_kernel<kOut2B>, grid, dim3(kThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace zp
