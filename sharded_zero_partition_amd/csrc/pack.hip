// pack.hip -- ragged-tensor bucket pack for gfx950.
//
// The constant-size buffers paragraph of the ZeRO explainer page (ZeRO-R)
// fuses many small gradient tensors into one fixed-size buffer so that the
// collective works on large messages.  Fill k of a bucket of B elements is
// the window [k*B, (k+1)*B) of the tensors laid back to back; past the end of
// the last tensor the bucket holds zeros.  The copy is bitwise.
//
// Design: the bucket is cut into 8-element (16-byte) vectors, so every store
// is an aligned 128-bit write, and the work is balanced over the bucket no
// matter how ragged the tensors are.  A wave owns a span of 512 U elements
// (U = 2) and lane l the vectors at 512 u + 8 l, so each store instruction
// writes 1 KiB contiguously.  The wave reads the source range of its span
// from a chunk index built at bind time (one entry per 2^shift >= 2048
// elements), through the scalar cache.  When the whole span lies in one
// tensor (almost always) the misalignment phase is wave-uniform: each lane
// loads one aligned 128-bit block per vector and takes the following block
// from its neighbour lane by cross-lane shuffle.  Otherwise each lane
// binary-searches the few candidate tensors, reads one aligned block (two and
// a funnel shift when misaligned) for a vector inside one tensor, and issues
// the loads of all U vectors before any is used; vectors that straddle
// tensors, touch a tensor edge or the end of the stream are gathered element
// by element.  No LDS staging: each wave's accesses are already contiguous.
// The first waves of a launch take the spans near tensor boundaries and the
// two ends of the fill's data (the work order of zp_internal.hpp), so that
// their slower path does not hold up the launch's end.
#include <hip/hip_ext.h>

#include "vec16.hpp"
#include "zp_internal.hpp"

namespace zp {
namespace {

constexpr int kPackThreads = 256;

// Element-by-element gather of up to nvalid elements from flat index g on,
// starting the source walk at index i; zeros past psi.
__device__ __forceinline__ u32x4 gather8(const PackSrc* __restrict__ src, int i, int64_t g,
                                         int nvalid, int64_t psi) {
    uint32_t w[4] = {0u, 0u, 0u, 0u};
#pragma unroll
    for (int e = 0; e < 8; ++e) {
        const int64_t ge = g + e;
        if (e < nvalid && ge < psi) {
            while (ge >= src[i].flat_off + src[i].len) ++i;
            const uint32_t val = ld2(src[i].ptr + (ge - src[i].flat_off));
            w[e >> 1] |= val << (16 * (e & 1));
        }
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

// Index of the source holding flat index g, searched in [lo, hi] only.
__device__ __forceinline__ int find_src_in(const PackSrc* __restrict__ src, int lo, int hi,
                                           int64_t g) {
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (src[mid].flat_off <= g)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

// Cooperative path of a full span inside one tensor: the misalignment phase
// ph is the same for the whole wave, so each lane loads a single aligned
// block per vector group from base0 on and takes the block after it from the
// next lane (the last lane of a group from the next group's first lane, and
// of the last group from one extra block read by the whole wave).
template <int U>
__device__ __forceinline__ void pack_coop(const PackLaunch& a, const uint16_t* base0, int ph, int64_t o_wave,
                                          int lane) {
    constexpr int64_t kSpan = 512 * U;
    u32x4 v[U];
#pragma unroll
    for (int u = 0; u < U; ++u)
        v[u] = ld16(base0 + 512 * u + 8 * lane);
    u32x4 extra = v[U - 1];
    if (ph) extra = ld16(base0 + kSpan);
#pragma unroll
    for (int u = 0; u < U; ++u) {
        u32x4 nxt;
        nxt.x = __shfl_down(v[u].x, 1);
        nxt.y = __shfl_down(v[u].y, 1);
        nxt.z = __shfl_down(v[u].z, 1);
        nxt.w = __shfl_down(v[u].w, 1);
        const u32x4 head = u + 1 < U ? v[u + 1 < U ? u + 1 : u] : extra;
        u32x4 first_of_next;
        first_of_next.x = __shfl(head.x, 0);
        first_of_next.y = __shfl(head.y, 0);
        first_of_next.z = __shfl(head.z, 0);
        first_of_next.w = __shfl(head.w, 0);
        if (lane == 63) nxt = first_of_next;
        const int64_t o = o_wave + 512 * u + 8 * lane;
        *reinterpret_cast<u32x4*>(a.bucket + o) = window8(v[u], nxt, ph);
    }
}

// Any span of the fill, starting at bucket element o_wave: the wave reads the
// source range of its span from the chunk index (two scalar loads); a full
// span inside one tensor takes the cooperative path, otherwise every lane
// finds its own source inside that range and issues the loads of all U
// vectors before any of them is used (up to 2U 16-byte loads in flight).
template <int U>
__device__ __forceinline__ void pack_general(const PackLaunch& a, int64_t o_wave, int lane) {
    constexpr int64_t kSpan = 512 * U;
    const int64_t g_wave = a.fill_base + o_wave;
    int lo = 0, hi = 0;
    if (g_wave < a.psi) {
        int64_t g_last = a.fill_base + min(o_wave + kSpan, a.bucket_elems) - 1;
        if (g_last >= a.psi) g_last = a.psi - 1;
        // sources of the span lie in [first[chunk(g_wave)], first[chunk(g_last) + 1]]
        lo = a.first[g_wave >> a.chunk_shift];
        hi = a.first[(g_last >> a.chunk_shift) + 1];
    }
    // when the whole span lies in one tensor its table entry is wave-uniform
    // and read once through the scalar cache
    const bool one_src = lo == hi;
    PackSrc uni = {nullptr, 0, 0};
    if (one_src && g_wave < a.psi) uni = a.src[lo];

    if (one_src && o_wave + kSpan <= a.bucket_elems && g_wave + kSpan <= a.psi) {
        const uint16_t* p0 = uni.ptr + (g_wave - uni.flat_off);
        const int ph = int((reinterpret_cast<uintptr_t>(p0) & 15) >> 1);
        const uint16_t* base0 = p0 - ph;
        const int64_t need = ph ? kSpan + 8 : kSpan;     // elements read from base0 on
        if (base0 >= uni.ptr && base0 + need <= uni.ptr + uni.len) {
            pack_coop<U>(a, base0, ph, o_wave, lane);
            return;
        }
    }
    int src_i[U];
    int mode[U];                 // 0 zeros, 1 aligned-window loads, 2 element gather
    const uint16_t* blk[U];      // first aligned 16-byte block
    int phase[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t o = o_wave + 512 * u + 8 * lane;
        const int64_t g = a.fill_base + o;
        src_i[u] = lo;
        mode[u] = 0;
        blk[u] = nullptr;
        phase[u] = 0;
        if (o < a.bucket_elems && g < a.psi) {
            const int i = one_src ? lo : find_src_in(a.src, lo, hi, g);
            src_i[u] = i;
            const PackSrc s = one_src ? uni : a.src[i];
            const int64_t rel = g - s.flat_off;
            mode[u] = 2;
            if (a.bucket_elems - o >= 8 && rel + 8 <= s.len) {
                const uint16_t* p = s.ptr + rel;
                const int ph = int((reinterpret_cast<uintptr_t>(p) & 15) >> 1);
                const uint16_t* base = p - ph;
                // the blocks read are [base, base + 8) and, when misaligned,
                // [base + 8, base + 16): both must lie inside the tensor
                if (ph == 0 || (base >= s.ptr && base + 16 <= s.ptr + s.len)) {
                    mode[u] = 1;
                    blk[u] = base;
                    phase[u] = ph;
                }
            }
        }
    }
    u32x4 lo_v[U], hi_v[U];
#pragma unroll
    for (int u = 0; u < U; ++u) {
        if (mode[u] == 1) {
            lo_v[u] = ld16(blk[u]);
            // aligned: read the same block twice rather than past its end
            hi_v[u] = ld16(blk[u] + (phase[u] ? 8 : 0));
        }
    }
#pragma unroll
    for (int u = 0; u < U; ++u) {
        const int64_t o = o_wave + 512 * u + 8 * lane;
        if (o >= a.bucket_elems) continue;
        const int64_t left = a.bucket_elems - o;
        const int nvalid = left < 8 ? int(left) : 8;
        u32x4 out = u32x4{0u, 0u, 0u, 0u};
        if (mode[u] == 1)
            out = window8(lo_v[u], hi_v[u], phase[u]);
        else if (mode[u] == 2)
            out = gather8(a.src, src_i[u], a.fill_base + o, nvalid, a.psi);
        if (nvalid == 8) {
            *reinterpret_cast<u32x4*>(a.bucket + o) = out;
        } else {
            const uint32_t w[4] = {out.x, out.y, out.z, out.w};
            for (int e = 0; e < nvalid; ++e)
                a.bucket[o + e] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

// Wave order as the launch plan sets it (PackLaunch::hard): the first n_hard
// waves take the two ends of the fill's data and the spans near tensor
// boundaries; wave n_hard + w takes span w: zeros past the data, else the
// cooperative path unless a boundary claims the span.  Lane l handles the U
// vectors at offsets 512 u + 8 l of its span, so each of the U store
// instructions covers 1 KiB of the bucket contiguously.
template <int U>
__global__ __launch_bounds__(kPackThreads) void pack_span_kernel(const PackLaunch a) {
    constexpr int64_t kSpan = 512 * U;
    static_assert(kSpan == kSpanElems, "the work order's span");
    const int lane = threadIdx.x & 63;
    // wave-uniform values live in scalar registers; the table reads below
    // then go through the scalar cache
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wave = int64_t(blockIdx.x) * (kPackThreads / 64) + wave_in_block;
    const bool in_order = a.hard.hard_per_b == 0;   // wave w takes span w
    if (!in_order && wave >= a.hard.n_hard) {
        const int64_t w = wave - a.hard.n_hard;
        if (w >= a.n_span) return;   // the whole wave leaves together
        const int64_t o_wave = w * kSpan;
        if (w >= a.n_data_span) {
            // past the end of the last tensor: zeros
#pragma unroll
            for (int u = 0; u < U; ++u) {
                const int64_t o = o_wave + 512 * u + 8 * lane;
                if (o + 8 <= a.bucket_elems) {
                    *reinterpret_cast<u32x4*>(a.bucket + o) = u32x4{0u, 0u, 0u, 0u};
                } else {
                    for (int64_t e = o; e < a.bucket_elems; ++e) a.bucket[e] = 0;
                }
            }
            return;
        }
        if (w == 0 || w == a.n_data_span - 1) return;   // hard waves 0 and 1
        const int64_t f = a.fill_base + o_wave;
        const PackSrc t = a.src[a.first[(f - 7) >> a.chunk_shift]];
        if (span_claimed(t.flat_off, t.len, f)) return;   // a hard wave's span
        const uint16_t* p0 = t.ptr + (f - t.flat_off);   // f - 7 >= t.flat_off
        const int ph = int((reinterpret_cast<uintptr_t>(p0) & 15) >> 1);
        const uint16_t* base0 = p0 - ph;
        const int64_t need = ph ? kSpan + 8 : kSpan;
        if (base0 >= t.ptr && base0 + need <= t.ptr + t.len)
            pack_coop<U>(a, base0, ph, o_wave, lane);
        else   // not reached: an unclaimed span lies inside t with 8 elements after it
            pack_general<U>(a, o_wave, lane);
        return;
    }
    const int64_t w = in_order ? (wave < a.n_span ? wave : -1)
                               : hard_wave_span(wave, a.n_data_span, a.fill_base, a.hard, a.chunk_shift,
                                                [&](int64_t i) { return i < a.n_src ? a.src[i].flat_off : a.psi; });
    if (w < 0) return;
    pack_general<U>(a, w * kSpan, lane);
}

constexpr int kPackSpanU = 2;

}  // namespace

hipError_t launch_pack(const PackLaunch& a, hipStream_t stream, const KernelEvents& ev) {
    const int64_t waves = a.hard.n_hard + a.n_span;
    if (waves > kMaxGridWaves) return hipErrorInvalidConfiguration;
    constexpr int64_t kWavesPerBlock = kPackThreads / 64;
    int64_t blocks = (waves + kWavesPerBlock - 1) / kWavesPerBlock;
    if (blocks < 1) blocks = 1;
    hipExtLaunchKernelGGL(pack_span_kernel<kPackSpanU>, dim3(unsigned(blocks)), dim3(kPackThreads), 0,
                          stream, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

}  // namespace zp
