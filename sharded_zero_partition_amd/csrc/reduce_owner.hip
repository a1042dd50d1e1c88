// reduce_owner.hip -- the owner's share of a bucketed gradient reduce, gfx950.
//
// In Stage 2 (P_os+g) of the ZeRO explainer page ("ZeRO: Memory Optimizations
// Toward Training Trillion Parameter Models", azimuth.plus) every rank ends up
// with only the reduced gradients of the partition it owns, and the ZeRO-R
// constant-size buffers paragraph streams the gradients through a fixed-size
// bucket.  This kernel is the local arithmetic of that exchange for one fill of
// the bucket and one owner: for each flat index g of the fill that the owner's
// shard holds, it sums the R ranks' fp16 values in fp32 (rank 0 first) and
// writes fp16(sum) into the owner's fp16 gradient shard.  The inputs are the R
// ranks' ragged gradient tensors themselves, so the pack and the reduce happen
// in one pass without materialising R buckets.
//
// Layout of the work: the owner's shard is cut into 8-element vectors on its
// own 16-byte grid, so every full vector is one aligned 128-bit store.  A wave
// owns 2 x 64 consecutive vectors (two 1 KiB store groups).  It reads the
// source range of its span from the chunk index built at bind time; when the
// span lies inside one tensor the tensor's offset, length and R addresses are
// wave-uniform (scalar loads), and so is each contribution's misalignment
// phase: every lane then loads one aligned block per vector group and takes
// the following block from its neighbour lane by cross-lane shuffle.
// Otherwise, for each vector whose 8 elements lie in one tensor, each
// contribution is read as aligned 16-byte blocks (funnel-shifted when
// misaligned); vectors at the range ends or across tensor boundaries go
// element by element.  HBM bytes per element: 2R read + 2 written.
#include "vec16.hpp"
#include "zp_internal.hpp"

namespace zp {
namespace {

constexpr int kThreads = 256;
constexpr int kU = 2;                     // vectors per lane
constexpr int64_t kSpanVec = 64 * kU;     // vectors per wave

// Last index i in [lo, hi] with off[i] <= g.
__device__ __forceinline__ int search(const int64_t* __restrict__ off, int lo, int hi, int64_t g) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (off[mid] <= g)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// fp32 sum over the contributions of the element at offset rel of source i.
template <int R>
__device__ __forceinline__ float sum1(const ReduceLaunch& a, int i, int64_t rel) {
    float s = h2f(ld2(a.ptr[i] + rel));
#pragma unroll
    for (int r = 1; r < R; ++r) s = s + h2f(ld2(a.ptr[int64_t(r) * a.n_src + i] + rel));
    return s;
}

// The next lane's block of each vector group: lane l < 63 takes lane l+1's
// block of group u, lane 63 the first block of group u+1 (or `extra`).
__device__ __forceinline__ u32x4 next_block(const u32x4 v[kU], int u, u32x4 extra, int lane) {
    u32x4 nxt;
    nxt.x = __shfl_down(v[u].x, 1);
    nxt.y = __shfl_down(v[u].y, 1);
    nxt.z = __shfl_down(v[u].z, 1);
    nxt.w = __shfl_down(v[u].w, 1);
    const u32x4 head = u + 1 < kU ? v[u + 1 < kU ? u + 1 : u] : extra;
    u32x4 first_of_next;
    first_of_next.x = __shfl(head.x, 0);
    first_of_next.y = __shfl(head.y, 0);
    first_of_next.z = __shfl(head.z, 0);
    first_of_next.w = __shfl(head.w, 0);
    return lane == 63 ? first_of_next : nxt;
}

// Cooperative span with a compile-time contribution count R.  The
// contributions go in groups of up to kGroup: all of a group's kU aligned
// blocks per lane (plus its extra blocks) are loaded before any is used, and
// the fp32 sums carry over from group to group in contribution order.  (All
// sixteen at once needs about 200 VGPRs and ran slower than two groups.)
constexpr int kGroup = 4;

template <int R>
__device__ __forceinline__ void coop_span(const ReduceLaunch& a, int src, int64_t rel0,
                                          int64_t kw, int mis, int lane) {
    constexpr int G = R < kGroup ? R : kGroup;
    float s[kU][8];
    int64_t dep = 0;   // 0; makes a group's addresses wait for the previous group's sums
#pragma unroll
    for (int r0 = 0; r0 < R; r0 += G) {
        u32x4 v[G][kU];
        u32x4 extra[G];
        int ph[G];
#pragma unroll
        for (int j = 0; j < G; ++j) {
            if (r0 + j >= R) break;
            const uint16_t* t = a.ptr[int64_t(r0 + j) * a.n_src + src];
            const uint16_t* p0 = t + rel0;
            ph[j] = int((reinterpret_cast<uintptr_t>(p0) & 15) >> 1);
            const uint16_t* b0 = p0 - ph[j] + dep;
#pragma unroll
            for (int u = 0; u < kU; ++u)
                v[j][u] = ld16_stream(b0 + 512 * u + 8 * lane);
            // aligned: re-read the last group's block rather than past the span
            extra[j] = ld16(b0 + (ph[j] ? 8 * kSpanVec : 512 * (kU - 1) + 8 * lane));
        }
#pragma unroll
        for (int u = 0; u < kU; ++u) {
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (r0 + j >= R) break;
                const u32x4 wv = window8(v[j][u], next_block(v[j], u, extra[j], lane), ph[j]);
                const uint32_t w[4] = {wv.x, wv.y, wv.z, wv.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = h2f(w[e >> 1] >> (16 * (e & 1)));
                    s[u][e] = r0 + j == 0 ? x : s[u][e] + x;
                }
            }
        }
        // The next group's loads may not start before this group's sums
        // exist: an empty asm statement takes a sum and yields `dep`, which
        // stays 0 but is opaque to the compiler, and the next addresses add it.
        if (r0 + G < R) asm volatile("" : "+v"(dep) : "v"(s[0][0]));
    }
#pragma unroll
    for (int u = 0; u < kU; ++u) {
        uint32_t o[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = f2h(s[u][2 * d]) | (f2h(s[u][2 * d + 1]) << 16);
        const int64_t jv = (kw + 64 * u + lane) * 8 - mis;
        __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]}, reinterpret_cast<u32x4*>(a.shard + jv));
    }
}

template <int R>
__global__ __launch_bounds__(kThreads) void reduce_owner_kernel(const ReduceLaunch a) {
    constexpr int nr = R;   // contributions (compile-time: every loop over them unrolls)
    const int lane = threadIdx.x & 63;
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wave = int64_t(blockIdx.x) * (kThreads / 64) + wave_in_block;
    // vector k covers shard positions [8k - mis, 8k - mis + 8)
    const int mis = int((reinterpret_cast<uintptr_t>(a.shard) >> 1) & 7);
    const int64_t j_lo = a.g_lo - a.base;
    const int64_t j_hi = a.g_hi - a.base;
    const int64_t k_lo = (j_lo + mis) >> 3;
    const int64_t k_end = ((j_hi - 1 + mis) >> 3) + 1;
    const int64_t kw = k_lo + wave * kSpanVec;
    if (kw >= k_end) return;   // the whole wave leaves together

    // sources of the wave's flat range
    const int64_t k_last = min(kw + kSpanVec, k_end) - 1;
    const int64_t jf = max(kw * 8 - mis, j_lo);
    const int64_t jl = min(k_last * 8 - mis + 8, j_hi) - 1;
    const int lo = a.first[(a.base + jf) >> a.chunk_shift];
    const int hi = a.first[((a.base + jl) >> a.chunk_shift) + 1];
    const bool one = lo == hi;
    int64_t one_off = 0, one_len = 0;
    if (one) {
        one_off = a.off[lo];
        one_len = a.len[lo];
    }

    // Cooperative path: a span of full vectors inside one tensor has one
    // misalignment phase per contribution for the whole wave, so each lane
    // loads one aligned block per vector group and takes the block after it
    // from the next lane (the last lane from the next group's first lane, or
    // from one extra block after the span).
    const bool full_span = kw * 8 - mis >= j_lo && (kw + kSpanVec) * 8 - mis <= j_hi;
    if (one && full_span) {
        const int64_t rel0 = a.base + kw * 8 - mis - one_off;    // >= 0, span inside the tensor
        bool in_bounds = true;
        for (int r = 0; r < nr; ++r) {
            const uint16_t* t = a.ptr[int64_t(r) * a.n_src + lo];
            const uint16_t* p0 = t + rel0;
            const int ph = int((reinterpret_cast<uintptr_t>(p0) & 15) >> 1);
            const uint16_t* b0 = p0 - ph;
            const int64_t need = ph ? 8 * kSpanVec + 8 : 8 * kSpanVec;
            in_bounds = in_bounds && b0 >= t && b0 + need <= t + one_len;
        }
        if (in_bounds) {
            // every contribution's loads are issued before the first shuffle
            coop_span<R>(a, lo, rel0, kw, mis, lane);
            return;
        }
    }

#pragma unroll
    for (int u = 0; u < kU; ++u) {
        const int64_t k = kw + 64 * u + lane;
        if (k >= k_end) continue;
        const int64_t jv = k * 8 - mis;
        const int64_t g0 = a.base + jv;
        if (jv >= j_lo && jv + 8 <= j_hi) {
            const int i = one ? lo : search(a.off, lo, hi, g0);
            const int64_t soff = one ? one_off : a.off[i];
            const int64_t slen = one ? one_len : a.len[i];
            const int64_t rel = g0 - soff;
            if (rel + 8 <= slen) {
                float s[8];
                int64_t dep = 0;   // as in coop_span: groups of kGroup contributions
#pragma unroll
                for (int r = 0; r < nr; ++r) {
                    const uint16_t* t = a.ptr[int64_t(r) * a.n_src + i + dep];
                    const u32x4 v = load8(t + rel, t, t + slen);
                    const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                    for (int e = 0; e < 8; ++e) {
                        const float x = h2f(w[e >> 1] >> (16 * (e & 1)));
                        s[e] = r == 0 ? x : s[e] + x;
                    }
                    if ((r + 1) % kGroup == 0 && r + 1 < nr) asm volatile("" : "+v"(dep) : "v"(s[0]));
                }
                uint32_t o[4];
#pragma unroll
                for (int d = 0; d < 4; ++d) o[d] = f2h(s[2 * d]) | (f2h(s[2 * d + 1]) << 16);
                *reinterpret_cast<u32x4*>(a.shard + jv) = u32x4{o[0], o[1], o[2], o[3]};
                continue;
            }
        }
        // range ends and tensor boundaries: element by element (rare; kept
        // rolled so that its loads do not set the kernel's register count)
#pragma unroll 1
        for (int e = 0; e < 8; ++e) {
            const int64_t j = jv + e;
            if (j < j_lo || j >= j_hi) continue;
            const int64_t g = a.base + j;
            const int i = search(a.off, lo, hi, g);
            a.shard[j] = uint16_t(f2h(sum1<R>(a, i, g - a.off[i])));
        }
    }
}

}  // namespace

hipError_t launch_reduce_owner(const ReduceLaunch& a, hipStream_t stream) {
    const int mis = int((reinterpret_cast<uintptr_t>(a.shard) >> 1) & 7);
    const int64_t j_lo = a.g_lo - a.base;
    const int64_t j_hi = a.g_hi - a.base;
    const int64_t nvec = ((j_hi - 1 + mis) >> 3) + 1 - ((j_lo + mis) >> 3);
    const int64_t waves = (nvec + kSpanVec - 1) / kSpanVec;
    int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks < 1) blocks = 1;
    const dim3 grid{unsigned(blocks)};
    switch (a.R) {
        case 1: hipLaunchKernelGGL(reduce_owner_kernel<1>, grid, dim3(kThreads), 0, stream, a); break;
        case 2: hipLaunchKernelGGL(reduce_owner_kernel<2>, grid, dim3(kThreads), 0, stream, a); break;
        case 3: hipLaunchKernelGGL(reduce_owner_kernel<3>, grid, dim3(kThreads), 0, stream, a); break;
        case 4: hipLaunchKernelGGL(reduce_owner_kernel<4>, grid, dim3(kThreads), 0, stream, a); break;
        case 5: hipLaunchKernelGGL(reduce_owner_kernel<5>, grid, dim3(kThreads), 0, stream, a); break;
        case 6: hipLaunchKernelGGL(reduce_owner_kernel<6>, grid, dim3(kThreads), 0, stream, a); break;
        case 7: hipLaunchKernelGGL(reduce_owner_kernel<7>, grid, dim3(kThreads), 0, stream, a); break;
        case 8: hipLaunchKernelGGL(reduce_owner_kernel<8>, grid, dim3(kThreads), 0, stream, a); break;
        case 9: hipLaunchKernelGGL(reduce_owner_kernel<9>, grid, dim3(kThreads), 0, stream, a); break;
        case 10: hipLaunchKernelGGL(reduce_owner_kernel<10>, grid, dim3(kThreads), 0, stream, a); break;
        case 11: hipLaunchKernelGGL(reduce_owner_kernel<11>, grid, dim3(kThreads), 0, stream, a); break;
        case 12: hipLaunchKernelGGL(reduce_owner_kernel<12>, grid, dim3(kThreads), 0, stream, a); break;
        case 13: hipLaunchKernelGGL(reduce_owner_kernel<13>, grid, dim3(kThreads), 0, stream, a); break;
        case 14: hipLaunchKernelGGL(reduce_owner_kernel<14>, grid, dim3(kThreads), 0, stream, a); break;
        case 15: hipLaunchKernelGGL(reduce_owner_kernel<15>, grid, dim3(kThreads), 0, stream, a); break;
        default: hipLaunchKernelGGL(reduce_owner_kernel<16>, grid, dim3(kThreads), 0, stream, a); break;
    }
    return hipGetLastError();
}

}  // namespace zp
