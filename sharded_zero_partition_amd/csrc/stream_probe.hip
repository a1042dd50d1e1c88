// stream_probe.hip -- achievable-bandwidth probes for the shard step, gfx950.
//
// A measurement aid, not part of the method: the kernels move the bytes of
// the fused shard step with none of its arithmetic, so their rate is the
// ceiling that the step's stream mix can reach on the machine, next to the
// 8 TB/s HBM peak.  The model-states paragraph of the ZeRO explainer page
// ("ZeRO: Memory Optimizations Toward Training Trillion Parameter Models",
// azimuth.plus) fixes what those bytes are: fp16 gradients, and an fp32
// master, momentum and variance per parameter; the step reads R fp16
// contributions and the three fp32 arrays and writes the three fp32 arrays
// and the fp16 parameter slot, 26 + 2R bytes per element.
//
//   step pattern  the step kernel's schedule and addressing exactly: one
//                 1024-element tile per wave over a full grid, lane l holding
//                 elements 4l .. 4l+3 of each 256-element group, non-temporal
//                 loads and stores; p, m, v are copied to the write set and
//                 the slot receives the XOR of the contributions' bits.
//   copy          the same tile-per-wave schedule on one read and one write
//                 stream of 16-byte blocks (4 KiB per wave).
//
// Every launch records a HIP event pair at its kernel's own start and end,
// and the call returns the mean kernel time over its launches.
#include <hip/hip_ext.h>
#include <hip/hip_runtime.h>

#include <cstdint>
#include <mutex>
#include <string>

#include "zero_probe.h"

namespace {

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));
typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kThreads = 256;
constexpr int kGroups = 4;                   // 256-element groups per tile
constexpr int64_t kTile = 256 * kGroups;     // elements per tile (one wave)
constexpr int kMaxR = 16;

thread_local std::string g_error;

int fail(int status, const std::string& msg) {
    g_error = msg;
    return status;
}

int fail_hip(hipError_t e, const char* what) {
    g_error = std::string(what) + ": " + hipGetErrorString(e);
    return ZERO_PROBE_ERR_HIP;
}

struct PatternArgs {
    const uint16_t* grad[kMaxR];
    const float* p;
    const float* m;
    const float* v;
    float* p_out;
    float* m_out;
    float* v_out;
    uint16_t* slot;      // 8-byte aligned
    int64_t n;
};

template <typename T>
__device__ __forceinline__ T ld(const T* p) {
    return __builtin_nontemporal_load(p);
}

template <typename T>
__device__ __forceinline__ void st(T* p, T v) {
    __builtin_nontemporal_store(v, p);
}

template <int R>
__global__ __launch_bounds__(kThreads) void step_pattern_kernel(const PatternArgs a) {
    const int lane = threadIdx.x & 63;
    const int64_t ntiles = a.n / kTile;
    const int64_t t = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
    if (t < ntiles) {
        u32x2 g[R][kGroups];
        f32x4 p[kGroups], m[kGroups], v[kGroups];
#pragma unroll
        for (int h = 0; h < kGroups; ++h) {
            const int64_t e = t * kTile + h * 256 + 4 * lane;
#pragma unroll
            for (int r = 0; r < R; ++r) g[r][h] = ld(reinterpret_cast<const u32x2*>(a.grad[r] + e));
            p[h] = ld(reinterpret_cast<const f32x4*>(a.p + e));
            m[h] = ld(reinterpret_cast<const f32x4*>(a.m + e));
            v[h] = ld(reinterpret_cast<const f32x4*>(a.v + e));
        }
#pragma unroll
        for (int h = 0; h < kGroups; ++h) {
            const int64_t e = t * kTile + h * 256 + 4 * lane;
            u32x2 x = g[0][h];
#pragma unroll
            for (int r = 1; r < R; ++r) x = x ^ g[r][h];
            st(reinterpret_cast<f32x4*>(a.p_out + e), p[h]);
            st(reinterpret_cast<f32x4*>(a.m_out + e), m[h]);
            st(reinterpret_cast<f32x4*>(a.v_out + e), v[h]);
            st(reinterpret_cast<u32x2*>(a.slot + e), x);
        }
    }
    // the elements past the last whole tile: block 0, one per thread per pass
    if (blockIdx.x == 0) {
        for (int64_t e = ntiles * kTile + threadIdx.x; e < a.n; e += kThreads) {
            uint16_t x = a.grad[0][e];
#pragma unroll
            for (int r = 1; r < R; ++r) x = uint16_t(x ^ a.grad[r][e]);
            a.p_out[e] = a.p[e];
            a.m_out[e] = a.m[e];
            a.v_out[e] = a.v[e];
            a.slot[e] = x;
        }
    }
}

// 16-byte blocks: wave w copies blocks [256 w, 256 (w + 1)), four per lane
// (lane l holds blocks 64 q + l); block 0 copies the last n mod 256 blocks.
__global__ __launch_bounds__(kThreads) void copy_kernel(const u32x4* __restrict__ src, u32x4* __restrict__ dst,
                                                        int64_t nblk) {
    const int lane = threadIdx.x & 63;
    const int64_t nw = nblk / 256;
    const int64_t w = int64_t(blockIdx.x) * (kThreads / 64) + (threadIdx.x >> 6);
    if (w < nw) {
        u32x4 x[4];
#pragma unroll
        for (int q = 0; q < 4; ++q) x[q] = ld(src + w * 256 + 64 * q + lane);
#pragma unroll
        for (int q = 0; q < 4; ++q) st(dst + w * 256 + 64 * q + lane, x[q]);
    }
    if (blockIdx.x == 0)
        for (int64_t b = nw * 256 + threadIdx.x; b < nblk; b += kThreads) dst[b] = src[b];
}

bool aligned(const void* p, uintptr_t a) { return (reinterpret_cast<uintptr_t>(p) & (a - 1)) == 0; }

// Per-thread event pair, created on first use on a device.
struct Events {
    hipEvent_t start = nullptr, stop = nullptr;
    int device = -1;
};
thread_local Events g_ev;

hipError_t events(hipEvent_t* s, hipEvent_t* e) {
    int dev = 0;
    hipError_t err = hipGetDevice(&dev);
    if (err != hipSuccess) return err;
    if (g_ev.device != dev) {
        if (g_ev.start) (void)hipEventDestroy(g_ev.start);
        if (g_ev.stop) (void)hipEventDestroy(g_ev.stop);
        g_ev = Events{};
        err = hipEventCreate(&g_ev.start);
        if (err == hipSuccess) err = hipEventCreate(&g_ev.stop);
        if (err != hipSuccess) return err;
        g_ev.device = dev;
    }
    *s = g_ev.start;
    *e = g_ev.stop;
    return hipSuccess;
}

// Runs `launch(start, stop)` `reps` times, each bracketed by the event pair at
// its kernel's start and end, and stores the mean kernel time in *ms.
template <class F>
int timed(F launch, int32_t reps, hipStream_t s, float* ms) {
    hipEvent_t e0, e1;
    hipError_t e = events(&e0, &e1);
    if (e != hipSuccess) return fail_hip(e, "probe events");
    double total = 0.0;
    for (int32_t i = 0; i < reps; ++i) {
        launch(e0, e1);
        e = hipGetLastError();
        if (e != hipSuccess) return fail_hip(e, "probe kernel launch");
        e = hipEventSynchronize(e1);
        float t = 0.0f;
        if (e == hipSuccess) e = hipEventElapsedTime(&t, e0, e1);
        if (e != hipSuccess) return fail_hip(e, "probe timing");
        total += t;
    }
    *ms = float(total / reps);
    return ZERO_PROBE_OK;
}

template <int R>
void launch_pattern(const PatternArgs& a, dim3 grid, hipStream_t s, hipEvent_t e0, hipEvent_t e1) {
    hipExtLaunchKernelGGL(step_pattern_kernel<R>, grid, dim3(kThreads), 0, s, e0, e1, 0, a);
}

}  // namespace

extern "C" int zero_probe_step_pattern(const uint16_t* const* grads, int32_t R, const float* p,
                                       const float* m, const float* v, float* p_out, float* m_out,
                                       float* v_out, uint16_t* slot, int64_t n, int32_t reps,
                                       void* stream, float* ms) {
    g_error.clear();
    if (!grads || !ms || R < 1 || R > kMaxR || n < 1 || reps < 1)
        return fail(ZERO_PROBE_ERR_INVALID_ARG, "zero_probe_step_pattern: bad argument");
    PatternArgs a{};
    for (int r = 0; r < R; ++r) {
        if (!grads[r] || !aligned(grads[r], 8)) return fail(ZERO_PROBE_ERR_INVALID_ARG, "contribution NULL or not 8-byte aligned");
        a.grad[r] = grads[r];
    }
    const void* arr[7] = {p, m, v, p_out, m_out, v_out, slot};
    for (int k = 0; k < 7; ++k)
        if (!arr[k] || !aligned(arr[k], k < 6 ? 16 : 8))
            return fail(ZERO_PROBE_ERR_INVALID_ARG, "array NULL or misaligned (fp32 16 bytes, slot 8)");
    if (n / kTile / (kThreads / 64) >= (int64_t(1) << 31))
        return fail(ZERO_PROBE_ERR_INVALID_ARG, "n too large for one launch");
    a.p = p;
    a.m = m;
    a.v = v;
    a.p_out = p_out;
    a.m_out = m_out;
    a.v_out = v_out;
    a.slot = slot;
    a.n = n;
    int64_t blocks = (n / kTile + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks < 1) blocks = 1;
    const dim3 grid{unsigned(blocks)};
    hipStream_t s = static_cast<hipStream_t>(stream);
    return timed([&](hipEvent_t e0, hipEvent_t e1) {
        switch (R) {
            case 1: launch_pattern<1>(a, grid, s, e0, e1); break;
            case 2: launch_pattern<2>(a, grid, s, e0, e1); break;
            case 3: launch_pattern<3>(a, grid, s, e0, e1); break;
            case 4: launch_pattern<4>(a, grid, s, e0, e1); break;
            case 5: launch_pattern<5>(a, grid, s, e0, e1); break;
            case 6: launch_pattern<6>(a, grid, s, e0, e1); break;
            case 7: launch_pattern<7>(a, grid, s, e0, e1); break;
            case 8: launch_pattern<8>(a, grid, s, e0, e1); break;
            case 9: launch_pattern<9>(a, grid, s, e0, e1); break;
            case 10: launch_pattern<10>(a, grid, s, e0, e1); break;
            case 11: launch_pattern<11>(a, grid, s, e0, e1); break;
            case 12: launch_pattern<12>(a, grid, s, e0, e1); break;
            case 13: launch_pattern<13>(a, grid, s, e0, e1); break;
            case 14: launch_pattern<14>(a, grid, s, e0, e1); break;
            case 15: launch_pattern<15>(a, grid, s, e0, e1); break;
            default: launch_pattern<16>(a, grid, s, e0, e1); break;
        }
    }, reps, s, ms);
}

extern "C" int zero_probe_copy(const void* src, void* dst, int64_t bytes, int32_t reps, void* stream,
                               float* ms) {
    g_error.clear();
    if (!src || !dst || !ms || bytes < 16 || (bytes & 15) || reps < 1 || !aligned(src, 16) ||
        !aligned(dst, 16))
        return fail(ZERO_PROBE_ERR_INVALID_ARG,
                    "zero_probe_copy: 16-byte aligned, non-NULL buffers and a positive multiple of 16 bytes");
    const int64_t nblk = bytes / 16;
    if (nblk / 256 / (kThreads / 64) >= (int64_t(1) << 31))
        return fail(ZERO_PROBE_ERR_INVALID_ARG, "copy too large for one launch");
    int64_t blocks = (nblk / 256 + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks < 1) blocks = 1;
    const dim3 grid{unsigned(blocks)};
    hipStream_t s = static_cast<hipStream_t>(stream);
    const u32x4* in = static_cast<const u32x4*>(src);
    u32x4* out = static_cast<u32x4*>(dst);
    return timed([&](hipEvent_t e0, hipEvent_t e1) {
        hipExtLaunchKernelGGL(copy_kernel, grid, dim3(kThreads), 0, s, e0, e1, 0, in, out, nblk);
    }, reps, s, ms);
}

extern "C" const char* zero_probe_last_error(void) { return g_error.c_str(); }
