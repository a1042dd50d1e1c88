// reduce_owner.hip -- the owner's share of a bucketed gradient reduce, and the
// owner step that feeds that reduce straight into the shard update, gfx950.
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
// owns 2 x 64 consecutive vectors (two 1 KiB store groups).  The first waves
// of a launch take the spans near tensor boundaries and the range's two ends
// (the work order of zp_internal.hpp), so that their slower path does not
// hold up the launch's end; every other wave reads one per-chunk record and
// either finds its span inside that record's tensor or leaves.  In a span
// inside one tensor the tensor's offset, length and R addresses are
// wave-uniform (scalar loads), and so is each contribution's misalignment
// phase: every lane then loads one aligned block per vector group and takes
// the following block from its neighbour lane by cross-lane shuffle.
// Otherwise the span's candidate tensors are staged in LDS; a vector whose 8
// elements lie in one tensor reads each contribution as aligned 16-byte
// blocks (funnel-shifted when misaligned), and vectors at the range ends or
// across tensor boundaries gather element by element.  HBM bytes per
// element: 2R read + 2 written.
//
// The owner step runs the same walk over the owner's whole real range and,
// in place of the fp16 store, the shard step's arithmetic (adam.hpp): the
// overflow check of each sum, Adam on the fp32 master, momentum and variance
// (read set -> write set) and the fp16 slot.  The Stage 2 reduce of the
// owner's partition and its Stage 1 update are then one pass, with no fp16
// gradient shard in between.  HBM bytes per element: 2R + 12 read, 12 + 2
// written.  A wave that saw a non-finite sum raises the flag word to the
// call's epoch; a one-thread kernel afterwards hands the decision to the
// host.
#include <hip/hip_ext.h>

#include <array>
#include <utility>

#include "adam.hpp"
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

typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef uint32_t u32x2 __attribute__((ext_vector_type(2)));

// What happens to the fp32 sums.  A span whose 2 x 64 vectors are all full
// and inside the range starts with `span_pre` (the loads the epilogue needs,
// issued before the table reads and the contributions' loads); when it also
// lies in one tensor it ends in `span_done`
// (the span's sums s[u][e] of shard positions j0 + 512 u + 8 lane + e).
// Other waves finish vector by vector: `pre` and `vec` for the 8-element
// vector at shard position jv, `elem` for a single element j.  `finish` is
// reached by every lane of every wave that did work.

// Reduce-to-owner: fp16 of the sum into the owner's fp16 gradient shard.
struct ToShard {
    using Launch = ReduceLaunch;
    struct SpanPre {};
    struct Pre {};
    __device__ static int mis(const Launch& a) {
        return int((reinterpret_cast<uintptr_t>(a.shard) >> 1) & 7);
    }
    __device__ static void span_pre(const Launch&, int64_t, int, SpanPre&) {}
    __device__ static void span_done(const Launch& a, int64_t j0, const float s[kU][8], const SpanPre&,
                                     int lane, bool&) {
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            uint32_t o[4];
#pragma unroll
            for (int d = 0; d < 4; ++d) o[d] = f2h(s[u][2 * d]) | (f2h(s[u][2 * d + 1]) << 16);
            __builtin_nontemporal_store(u32x4{o[0], o[1], o[2], o[3]},
                                        reinterpret_cast<u32x4*>(a.shard + j0 + 512 * u + 8 * lane));
        }
    }
    __device__ static void pre(const Launch&, int64_t, Pre&) {}
    __device__ static void vec(const Launch& a, int64_t jv, const float s[8], const Pre&, bool&) {
        uint32_t o[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) o[d] = f2h(s[2 * d]) | (f2h(s[2 * d + 1]) << 16);
        *reinterpret_cast<u32x4*>(a.shard + jv) = u32x4{o[0], o[1], o[2], o[3]};
    }
    __device__ static void elem(const Launch& a, int64_t j, float s, bool&) {
        a.shard[j] = uint16_t(f2h(s));
    }
    // the elements of the vector at jv whose bit is set in mask
    __device__ static void part(const Launch& a, int64_t jv, const float s[8], unsigned mask, bool&) {
#pragma unroll
        for (int e = 0; e < 8; ++e)
            if ((mask >> e) & 1) a.shard[jv + e] = uint16_t(f2h(s[e]));
    }
    __device__ static void finish(const Launch&, bool) {}
};

// Owner step: the shard step's arithmetic on element j of the owner's shard
// (ping-pong: read set *_in, write set *_out and the fp16 slot).
//
// In a cooperative span lane l holds the sums of elements 8 l .. 8 l + 7 of
// each 512-element group, but an fp32 access with that mapping covers only
// half of every 64-byte run it touches, and such non-temporal stores cost
// about 1.5x their bytes in HBM writes (measured).  So the sums go through
// LDS (16 KiB per block, each wave its own 4 KiB) and come back as 4
// consecutive elements per lane, 256 q + 4 l .. + 3 for q = 0..3: every
// fp32 load and store instruction then covers 1 KiB contiguously, and the
// fp16 slot 512 bytes.
struct ToAdam {
    using Launch = OwnerLaunch;
    struct SpanPre {
        f32x4 p[4], m[4], v[4];
    };
    struct Pre {
        f32x4 p[2], m[2], v[2];
    };
    __device__ static int mis(const Launch&) { return 0; }   // p, m, v are 16-byte aligned
    __device__ static void span_pre(const Launch& a, int64_t j0, int lane, SpanPre& q) {
        const StepLaunch& c = a.st;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t e = j0 + 256 * k + 4 * lane;
            q.p[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(c.p_in + e));
            q.m[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(c.m_in + e));
            q.v[k] = __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(c.v_in + e));
        }
    }
    __device__ static void span_done(const Launch& a, int64_t j0, const float s[kU][8], const SpanPre& q,
                                     int lane, bool& bad) {
        static_assert(kU == 2, "the transpose below assumes two 512-element groups");
        __shared__ f32x4 lds[kThreads / 64][256];
        f32x4* mine = lds[threadIdx.x >> 6];
#pragma unroll
        for (int u = 0; u < kU; ++u) {
            mine[128 * u + 2 * lane] = f32x4{s[u][0], s[u][1], s[u][2], s[u][3]};
            mine[128 * u + 2 * lane + 1] = f32x4{s[u][4], s[u][5], s[u][6], s[u][7]};
        }
        // only this wave touches its slice: LDS operations of one wave
        // complete in order, the fences keep the compiler from reordering
        __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
        __builtin_amdgcn_wave_barrier();
        __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
        const StepLaunch& c = a.st;
        const uintptr_t slot_phase = reinterpret_cast<uintptr_t>(c.out16 + j0) & 7;   // wave-uniform
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const f32x4 t = mine[64 * k + lane];
            const float sk[4] = {t.x, t.y, t.z, t.w};
            float p[4] = {q.p[k].x, q.p[k].y, q.p[k].z, q.p[k].w};
            float m[4] = {q.m[k].x, q.m[k].y, q.m[k].z, q.m[k].w};
            float v[4] = {q.v[k].x, q.v[k].y, q.v[k].z, q.v[k].w};
#pragma unroll
            for (int e = 0; e < 4; ++e) {
                bad |= not_finite(sk[e]);
                adam_element(c, sk[e], p[e], m[e], v[e]);
            }
            const int64_t e0 = j0 + 256 * k + 4 * lane;
            __builtin_nontemporal_store(f32x4{p[0], p[1], p[2], p[3]}, reinterpret_cast<f32x4*>(c.p_out + e0));
            __builtin_nontemporal_store(f32x4{m[0], m[1], m[2], m[3]}, reinterpret_cast<f32x4*>(c.m_out + e0));
            __builtin_nontemporal_store(f32x4{v[0], v[1], v[2], v[3]}, reinterpret_cast<f32x4*>(c.v_out + e0));
            const uint32_t w0 = f2h(p[0]) | (f2h(p[1]) << 16);
            const uint32_t w1 = f2h(p[2]) | (f2h(p[3]) << 16);
            uint16_t* dst = c.out16 + e0;
            if (slot_phase == 0) {
                __builtin_nontemporal_store(u32x2{w0, w1}, reinterpret_cast<u32x2*>(dst));
            } else if ((slot_phase & 3) == 0) {
                __builtin_nontemporal_store(w0, reinterpret_cast<uint32_t*>(dst));
                __builtin_nontemporal_store(w1, reinterpret_cast<uint32_t*>(dst + 2));
            } else {
                dst[0] = uint16_t(w0);
                dst[1] = uint16_t(w0 >> 16);
                dst[2] = uint16_t(w1);
                dst[3] = uint16_t(w1 >> 16);
            }
        }
    }
    // vector by vector (waves at the range ends or over tensor boundaries)
    __device__ static void pre(const Launch& a, int64_t jv, Pre& q) {
        const StepLaunch& c = a.st;
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            q.p[h] = *reinterpret_cast<const f32x4*>(c.p_in + jv + 4 * h);
            q.m[h] = *reinterpret_cast<const f32x4*>(c.m_in + jv + 4 * h);
            q.v[h] = *reinterpret_cast<const f32x4*>(c.v_in + jv + 4 * h);
        }
    }
    __device__ static void vec(const Launch& a, int64_t jv, const float s[8], const Pre& q, bool& bad) {
        const StepLaunch& c = a.st;
        float p[8] = {q.p[0].x, q.p[0].y, q.p[0].z, q.p[0].w, q.p[1].x, q.p[1].y, q.p[1].z, q.p[1].w};
        float m[8] = {q.m[0].x, q.m[0].y, q.m[0].z, q.m[0].w, q.m[1].x, q.m[1].y, q.m[1].z, q.m[1].w};
        float v[8] = {q.v[0].x, q.v[0].y, q.v[0].z, q.v[0].w, q.v[1].x, q.v[1].y, q.v[1].z, q.v[1].w};
#pragma unroll
        for (int k = 0; k < 8; ++k) {
            bad |= not_finite(s[k]);
            adam_element(c, s[k], p[k], m[k], v[k]);
        }
#pragma unroll
        for (int h = 0; h < 2; ++h) {
            *reinterpret_cast<f32x4*>(c.p_out + jv + 4 * h) = f32x4{p[4 * h], p[4 * h + 1], p[4 * h + 2], p[4 * h + 3]};
            *reinterpret_cast<f32x4*>(c.m_out + jv + 4 * h) = f32x4{m[4 * h], m[4 * h + 1], m[4 * h + 2], m[4 * h + 3]};
            *reinterpret_cast<f32x4*>(c.v_out + jv + 4 * h) = f32x4{v[4 * h], v[4 * h + 1], v[4 * h + 2], v[4 * h + 3]};
        }
        // the slot may be only 2-byte aligned; jv is a multiple of 8, so every
        // lane of the wave takes the same branch
        uint32_t w[4];
#pragma unroll
        for (int d = 0; d < 4; ++d) w[d] = f2h(p[2 * d]) | (f2h(p[2 * d + 1]) << 16);
        uint16_t* dst = c.out16 + jv;
        const uintptr_t x = reinterpret_cast<uintptr_t>(dst);
        if ((x & 15) == 0) {
            *reinterpret_cast<u32x4*>(dst) = u32x4{w[0], w[1], w[2], w[3]};
        } else if ((x & 7) == 0) {
            *reinterpret_cast<u32x2*>(dst) = u32x2{w[0], w[1]};
            *reinterpret_cast<u32x2*>(dst + 4) = u32x2{w[2], w[3]};
        } else if ((x & 3) == 0) {
#pragma unroll
            for (int d = 0; d < 4; ++d) *reinterpret_cast<uint32_t*>(dst + 2 * d) = w[d];
        } else {
#pragma unroll
            for (int e = 0; e < 8; ++e) dst[e] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
        }
    }
    __device__ static void elem(const Launch& a, int64_t j, float s, bool& bad) {
        const StepLaunch& c = a.st;
        bad |= not_finite(s);
        float p = c.p_in[j], m = c.m_in[j], v = c.v_in[j];
        adam_element(c, s, p, m, v);
        c.p_out[j] = p;
        c.m_out[j] = m;
        c.v_out[j] = v;
        c.out16[j] = uint16_t(f2h(p));
    }
    // the elements of the vector at jv whose bit is set in mask, every load
    // issued before the first is used
    __device__ static void part(const Launch& a, int64_t jv, const float s[8], unsigned mask, bool& bad) {
        const StepLaunch& c = a.st;
        float p[8], m[8], v[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            const bool in = (mask >> e) & 1;
            p[e] = in ? c.p_in[jv + e] : 0.0f;
            m[e] = in ? c.m_in[jv + e] : 0.0f;
            v[e] = in ? c.v_in[jv + e] : 0.0f;
        }
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            if (!((mask >> e) & 1)) continue;
            bad |= not_finite(s[e]);
            adam_element(c, s[e], p[e], m[e], v[e]);
            c.p_out[jv + e] = p[e];
            c.m_out[jv + e] = m[e];
            c.v_out[jv + e] = v[e];
            c.out16[jv + e] = uint16_t(f2h(p[e]));
        }
    }
    __device__ static void finish(const Launch& a, bool bad) {
        const unsigned long long ballot = __ballot(bad);
        if (ballot != 0ull && (threadIdx.x & 63) == 0) atomicMax(a.st.flag, a.st.epoch);
    }
};

// Cooperative span with a compile-time contribution count R.  The
// contributions go in groups of up to kGroup: all of a group's kU aligned
// blocks per lane (plus its extra blocks) are loaded before any is used, and
// the fp32 sums carry over from group to group in contribution order.  (All
// sixteen at once needs about 200 VGPRs and ran slower than two groups.)
constexpr int kGroup = 4;

template <int R, class Epi>
__device__ __forceinline__ void coop_span(const typename Epi::Launch& a, const uint16_t* const (&src)[R], int64_t rel0,
                                          int64_t kw, int mis, int lane, bool& bad,
                                          const typename Epi::SpanPre& pre) {
    constexpr int G = R < kGroup ? R : kGroup;
    const int64_t j0 = kw * 8 - mis;
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
            const uint16_t* t = src[r0 + j];
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
    Epi::span_done(a, j0, s, pre, lane, bad);
}

// Spans off the cooperative path: spans that hold tensor boundaries, and
// spans at the ends of the owner's range.  Their elements used to wait on a
// chain of dependent reads each (a binary search over the table, the
// tensor's entry, its address, then the data, one element after another); a
// wave like that lives many times longer than the others, and as the last
// wave of a launch it holds up the launch's end.  So the span's candidate
// tensors (at most kStage of them) are staged first: lane l reads the start,
// end and R addresses of tensor lo + l into the wave's LDS slice, all at
// once.  Each vector then finds its tensor in LDS; a vector inside one tensor
// reads aligned blocks, and any other vector finds each element's tensor in
// LDS and issues all eight elements' loads of a contribution together.
// One per-chunk record of the reduce tables (layout: chunk_rec_bytes).
template <int R>
struct alignas(16) ChunkRec {
    int64_t off;
    int64_t len;
    int32_t idx;
    int32_t pad;
    const uint16_t* ptr[R];
};
static_assert(sizeof(ChunkRec<1>) == chunk_rec_bytes(1) && sizeof(ChunkRec<2>) == chunk_rec_bytes(2) &&
                  sizeof(ChunkRec<5>) == chunk_rec_bytes(5) && sizeof(ChunkRec<16>) == chunk_rec_bytes(16),
              "record layout");

template <int R>
struct Stage {
    static constexpr int kMax = R <= 4 ? 64 : 16;   // candidate tensors per span
    int64_t off[kMax];
    int64_t end[kMax];
    const uint16_t* ptr[R][kMax];
};

template <int R, class Epi>
__device__ __forceinline__ void staged_vectors(const typename Epi::Launch& a, int lo, int ncand, int64_t kw,
                                               int64_t k_end, int mis, int64_t j_lo, int64_t j_hi, int lane,
                                               int wave_in_block, bool& bad) {
    __shared__ Stage<R> stage[kThreads / 64];
    Stage<R>& st = stage[wave_in_block];
    if (lane < ncand) {
        const int64_t o = a.off[lo + lane];
        st.off[lane] = o;
        st.end[lane] = o + a.len[lo + lane];
#pragma unroll
        for (int r = 0; r < R; ++r) st.ptr[r][lane] = a.ptr[int64_t(r) * a.n_src + lo + lane];
    }
    // only this wave touches its slice: LDS operations of one wave complete
    // in order, the fences keep the compiler from reordering
    __builtin_amdgcn_fence(__ATOMIC_RELEASE, "wavefront");
    __builtin_amdgcn_wave_barrier();
    __builtin_amdgcn_fence(__ATOMIC_ACQUIRE, "wavefront");
#pragma unroll 1
    for (int u = 0; u < kU; ++u) {
        const int64_t k = kw + 64 * u + lane;
        if (k >= k_end) continue;
        const int64_t jv = k * 8 - mis;
        const int64_t g0 = a.base + jv;
        // the candidate holding g0 (the span's first in-range position is in
        // candidate 0, so g0 < off[0] only for a vector that starts before
        // the range, whose elements there are not read)
        int i0 = 0;
        for (int step = Stage<R>::kMax / 2; step > 0; step >>= 1)   // binary search in LDS
            if (i0 + step < ncand && st.off[i0 + step] <= g0) i0 += step;
        const bool whole = jv >= j_lo && jv + 8 <= j_hi;
        if (whole && g0 >= st.off[i0] && g0 + 8 <= st.end[i0]) {
            const int64_t soff = st.off[i0];
            const int64_t slen = st.end[i0] - soff;
            const int64_t rel = g0 - soff;
            typename Epi::Pre pre;
            Epi::pre(a, jv, pre);
            float s[8];
            int64_t dep = 0;   // as in coop_span: groups of kGroup contributions
#pragma unroll
            for (int r = 0; r < R; ++r) {
                const uint16_t* t = st.ptr[r][i0] + dep;
                const u32x4 v = load8(t + rel, t, t + slen);
                const uint32_t w[4] = {v.x, v.y, v.z, v.w};
#pragma unroll
                for (int e = 0; e < 8; ++e) {
                    const float x = h2f(w[e >> 1] >> (16 * (e & 1)));
                    s[e] = r == 0 ? x : s[e] + x;
                }
                if ((r + 1) % kGroup == 0 && r + 1 < R) asm volatile("" : "+v"(dep) : "v"(s[0]));
            }
            Epi::vec(a, jv, s, pre, bad);
            continue;
        }
        // across boundaries or at a range end: each element's candidate from
        // LDS, then per contribution all eight elements' loads at once
        unsigned mask = 0;
        int cand[8];
        int ie = i0;
#pragma unroll
        for (int e = 0; e < 8; ++e) {
            while (ie + 1 < ncand && st.off[ie + 1] <= g0 + e) ++ie;
            cand[e] = ie;
            if (jv + e >= j_lo && jv + e < j_hi) mask |= 1u << e;
        }
        int64_t rel[8];
#pragma unroll
        for (int e = 0; e < 8; ++e) rel[e] = g0 + e - st.off[cand[e]];
        // contributions in groups of kGroup, each group's loads all issued
        // before any is used; the sums carry over in contribution order
        constexpr int G = R < kGroup ? R : kGroup;
        float s[8];
        int64_t dep = 0;   // as in coop_span: the next group waits for this one's sums
#pragma unroll
        for (int r0 = 0; r0 < R; r0 += G) {
            uint32_t x[G][8];
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (r0 + j >= R) break;
#pragma unroll
                for (int e = 0; e < 8; ++e)
                    x[j][e] = (mask >> e) & 1 ? ld2(st.ptr[r0 + j][cand[e]] + rel[e] + dep) : 0u;
            }
#pragma unroll
            for (int j = 0; j < G; ++j) {
                if (r0 + j >= R) break;
#pragma unroll
                for (int e = 0; e < 8; ++e) s[e] = r0 + j == 0 ? h2f(x[j][e]) : s[e] + h2f(x[j][e]);
            }
            if (r0 + G < R) asm volatile("" : "+v"(dep) : "v"(s[0]));
        }
        if (mask == 0xFFu) {
            typename Epi::Pre pre;
            Epi::pre(a, jv, pre);
            Epi::vec(a, jv, s, pre, bad);
        } else {
            Epi::part(a, jv, s, mask, bad);
        }
    }
}

// The reads of a cooperative span at offset rel0 of a tensor of len
// elements stay inside the tensor for every contribution (the blocks from
// the aligned block holding rel0 on, plus one more when misaligned).
template <int R>
__device__ __forceinline__ bool coop_in_bounds(const uint16_t* const (&ptr)[R], int64_t rel0, int64_t len) {
    bool ok = true;
#pragma unroll
    for (int r = 0; r < R; ++r) {
        const uint16_t* t = ptr[r];
        const uint16_t* p0 = t + rel0;
        const int ph = int((reinterpret_cast<uintptr_t>(p0) & 15) >> 1);
        const uint16_t* b0 = p0 - ph;
        const int64_t need = ph ? 8 * kSpanVec + 8 : 8 * kSpanVec;
        ok = ok && b0 >= t && b0 + need <= t + len;
    }
    return ok;
}

// Any span, first vector kw: the cooperative path when the span is whole and
// inside one tensor, else the staged or the per-vector path.
template <int R, class Epi>
__device__ __forceinline__ void general_span(const typename Epi::Launch& a, int64_t kw, int64_t k_end, int mis,
                                             int64_t j_lo, int64_t j_hi, int lane, int wave_in_block, bool& bad) {
    constexpr int nr = R;   // contributions (compile-time: every loop over them unrolls)
    // A span of full vectors starts its epilogue's own loads (p, m, v for the
    // owner step) before the table reads below: their addresses need only the
    // span's position, so their latency overlaps the dependent table reads.
    const bool full_span = kw * 8 - mis >= j_lo && (kw + kSpanVec) * 8 - mis <= j_hi;
    typename Epi::SpanPre pre;
    if (full_span) Epi::span_pre(a, kw * 8 - mis, lane, pre);

    // sources of the wave's flat range
    const int64_t k_last = min(kw + kSpanVec, k_end) - 1;
    const int64_t jf = max(kw * 8 - mis, j_lo);
    const int64_t jl = min(k_last * 8 - mis + 8, j_hi) - 1;
    // The record of the chunk holding the span's first position carries the
    // entries of the tensor holding that chunk's start (offset, length, index
    // and R addresses), and the chunk index gives the last candidate: two
    // independent reads, so the tables cost one latency before the data
    // loads.  (A chain of table reads -- chunk index, then the tensor's
    // entries, then its addresses -- meets cold lines at the start and the
    // end of every launch and added a few microseconds to each.)
    const ChunkRec<R>& rec = reinterpret_cast<const ChunkRec<R>*>(a.rec)[(a.base + jf) >> a.chunk_shift];
    const int hi = a.first[((a.base + jl) >> a.chunk_shift) + 1];
    const int lo = rec.idx;
    const int64_t one_off = rec.off;
    const int64_t one_len = rec.len;
    const uint16_t* one_ptr[R];
#pragma unroll
    for (int r = 0; r < R; ++r) one_ptr[r] = rec.ptr[r];
    // keeps the compiler from sinking the address loads into the branches
    // below, behind a second wait (after every load: a load placed after
    // such a statement could no longer go through the scalar cache)
#pragma unroll
    for (int r = 0; r < R; ++r) asm volatile("" ::"s"(one_ptr[r]));
    const bool one = lo == hi;

    // Cooperative path: a span of full vectors inside one tensor has one
    // misalignment phase per contribution for the whole wave, so each lane
    // loads one aligned block per vector group and takes the block after it
    // from the next lane (the last lane from the next group's first lane, or
    // from one extra block after the span).
    if (one && full_span) {
        const int64_t rel0 = a.base + kw * 8 - mis - one_off;    // >= 0, span inside the tensor
        if (coop_in_bounds<R>(one_ptr, rel0, one_len)) {
            // every contribution's loads are issued before the first shuffle
            coop_span<R, Epi>(a, one_ptr, rel0, kw, mis, lane, bad, pre);
            return;
        }
    }

    if (hi - lo < Stage<R>::kMax) {
        staged_vectors<R, Epi>(a, lo, hi - lo + 1, kw, k_end, mis, j_lo, j_hi, lane, wave_in_block, bad);
        return;
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
                typename Epi::Pre pre;
                Epi::pre(a, jv, pre);
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
                Epi::vec(a, jv, s, pre, bad);
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
            Epi::elem(a, j, sum1<R>(a, i, g - a.off[i]), bad);
        }
    }
}

static_assert(kSpanVec == kSpanVecs, "one span geometry for host and device");

// The wave's work, in the order the launch plan sets (ReduceLaunch): the
// first n_hard waves take the two ends of the range and the spans near
// tensor boundaries, the rest one span each, leaving at once when a boundary
// claims that span.
template <int R, class Epi>
__device__ __forceinline__ void owner_body(const typename Epi::Launch& a) {
    const int lane = threadIdx.x & 63;
    const int wave_in_block = __builtin_amdgcn_readfirstlane(threadIdx.x >> 6);
    const int64_t wave = int64_t(blockIdx.x) * (kThreads / 64) + wave_in_block;
    const int mis = Epi::mis(a);
    const int64_t j_lo = a.g_lo - a.base;
    const int64_t j_hi = a.g_hi - a.base;
    const SpanGeometry geo = span_geometry(a.base, j_lo, j_hi, mis);
    bool bad = false;

    const bool in_order = a.hard.hard_per_b == 0;   // wave w takes span w
    if (!in_order && wave >= a.hard.n_hard) {
        // interior span w: whole and inside the range
        const int64_t w = wave - a.hard.n_hard;
        if (w < 1 || w >= geo.n_span - 1) return;   // the whole wave leaves together
        const int64_t kw = geo.k_lo + w * kSpanVec;
        const int64_t f = geo.span0 + w * kSpanElems;
        // the epilogue's own loads (p, m, v for the owner step) need only the
        // span's position: issued first, their latency overlaps the record's
        typename Epi::SpanPre pre;
        Epi::span_pre(a, kw * 8 - mis, lane, pre);
        const ChunkRec<R>& rec = reinterpret_cast<const ChunkRec<R>*>(a.rec)[(f - 7) >> a.chunk_shift];
        const int64_t one_off = rec.off;
        const int64_t one_len = rec.len;
        const uint16_t* one_ptr[R];
#pragma unroll
        for (int r = 0; r < R; ++r) one_ptr[r] = rec.ptr[r];
        // keeps the address loads together, ahead of the branches below
#pragma unroll
        for (int r = 0; r < R; ++r) asm volatile("" ::"s"(one_ptr[r]));
        if (span_claimed(one_off, one_len, f)) return;   // a hard wave's span
        const int64_t rel0 = f - one_off;   // >= 7: the record's tensor starts by f - 7
        if (coop_in_bounds<R>(one_ptr, rel0, one_len)) {
            coop_span<R, Epi>(a, one_ptr, rel0, kw, mis, lane, bad, pre);
        } else {
            // Not reached (an unclaimed span lies inside the record's tensor,
            // with 7 elements before it and 8 after it); kept so that no read
            // can leave a tensor: element by element, each found by search.
#pragma unroll 1
            for (int e = 0; e < int(kSpanElems / 64); ++e) {
                const int64_t j = kw * 8 - mis + 64 * e + lane;
                const int64_t g = a.base + j;
                const int i = search(a.off, 0, a.n_src - 1, g);
                Epi::elem(a, j, sum1<R>(a, i, g - a.off[i]), bad);
            }
        }
        Epi::finish(a, bad);
        return;
    }

    const int64_t w = in_order ? (wave < geo.n_span ? wave : -1)
                               : hard_wave_span(wave, geo.n_span, geo.span0, a.hard, a.chunk_shift,
                                                [&](int64_t i) { return a.off[i]; });
    if (w < 0) return;
    general_span<R, Epi>(a, geo.k_lo + w * kSpanVec, geo.k_end, mis, j_lo, j_hi, lane, wave_in_block, bad);
    Epi::finish(a, bad);
}

template <int R>
__global__ __launch_bounds__(kThreads) void reduce_owner_kernel(const ReduceLaunch a) {
    owner_body<R, ToShard>(a);
}

template <int R>
__global__ __launch_bounds__(kThreads) void owner_step_kernel(const OwnerLaunch a) {
    owner_body<R, ToAdam>(a);
}

// The shard's padding, positions [j0, n) of an owner step: no contribution
// reaches it, so each element takes the Adam step with a zero gradient sum,
// as the dense shard step does over zero-filled contributions.  Padding is
// at most N * A - 1 elements except on a rank that holds only padding.
__global__ __launch_bounds__(kThreads) void owner_pad_kernel(const StepLaunch a, int64_t j0) {
    const int64_t stride = int64_t(gridDim.x) * kThreads;
    for (int64_t j = j0 + int64_t(blockIdx.x) * kThreads + threadIdx.x; j < a.n; j += stride) {
        float p = a.p_in[j], m = a.m_in[j], v = a.v_in[j];
        adam_element(a, 0.0f, p, m, v);
        a.p_out[j] = p;
        a.m_out[j] = m;
        a.v_out[j] = v;
        a.out16[j] = uint16_t(f2h(p));
    }
}

// One thread, launched after the owner step on its stream: copies the pass's
// decision from the flag word into the pinned host word the host polls.
__global__ void publish_flag_kernel(const uint32_t* flag, uint32_t epoch, unsigned long long* host_word) {
    const uint32_t f = __hip_atomic_load(flag, __ATOMIC_RELAXED, __HIP_MEMORY_SCOPE_AGENT);
    const unsigned long long word = (static_cast<unsigned long long>(epoch) << 1) | (f == epoch ? 1ull : 0ull);
    __hip_atomic_store(host_word, word, __ATOMIC_RELEASE, __HIP_MEMORY_SCOPE_SYSTEM);
}

// The kernels for R = 1..16, indexed by R - 1.
template <int... I>
std::array<void (*)(ReduceLaunch), sizeof...(I)> reduce_kernels(std::integer_sequence<int, I...>) {
    return {{&reduce_owner_kernel<I + 1>...}};
}
template <int... I>
std::array<void (*)(OwnerLaunch), sizeof...(I)> owner_kernels(std::integer_sequence<int, I...>) {
    return {{&owner_step_kernel<I + 1>...}};
}
const auto kReduceKernels = reduce_kernels(std::make_integer_sequence<int, kMaxReduceRanks>{});
const auto kOwnerKernels = owner_kernels(std::make_integer_sequence<int, kMaxReduceRanks>{});

// Workgroups of the launch plan: n_hard waves, then one wave per span.
dim3 plan_grid(const ReduceLaunch& a) {
    const int64_t waves = a.hard.n_hard + a.n_span;   // <= kMaxGridWaves (checked by the launchers)
    int64_t blocks = (waves + kThreads / 64 - 1) / (kThreads / 64);
    if (blocks < 1) blocks = 1;
    return dim3{unsigned(blocks)};
}

}  // namespace

hipError_t launch_reduce_owner(const ReduceLaunch& a, hipStream_t stream, const KernelEvents& ev) {
    if (a.hard.n_hard + a.n_span > kMaxGridWaves) return hipErrorInvalidConfiguration;
    const dim3 grid = plan_grid(a);
    if (a.R < 1 || a.R > kMaxReduceRanks) return hipErrorInvalidValue;   // checked at bind time
    hipExtLaunchKernelGGL(kReduceKernels[a.R - 1], grid, dim3(kThreads), 0, stream, ev.start, ev.stop, 0, a);
    return hipGetLastError();
}

namespace {

// The owner step's main pass over the real elements [g_lo, g_hi).
void launch_owner_real(const OwnerLaunch& a, hipStream_t stream, const KernelEvents& ev) {
    const dim3 grid = plan_grid(a);
    hipExtLaunchKernelGGL(kOwnerKernels[a.R - 1], grid, dim3(kThreads), 0, stream, ev.start, ev.stop, 0, a);
}

}  // namespace

hipError_t launch_owner_step(const OwnerLaunch& a, hipStream_t stream, const KernelEvents& ev) {
    if (a.hard.n_hard + a.n_span > kMaxGridWaves) return hipErrorInvalidConfiguration;
    if (a.R < 1 || a.R > kMaxReduceRanks) return hipErrorInvalidValue;   // checked at bind time
    // the shard is [0, a.st.n): its real elements first, then its padding
    const int64_t n_real = a.g_hi - a.g_lo;
    const bool pad = a.st.n > n_real;
    if (n_real > 0) {
        launch_owner_real(a, stream, KernelEvents{ev.start, pad ? nullptr : ev.stop});
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    if (pad) {
        int64_t blocks = (a.st.n - n_real + kThreads - 1) / kThreads;
        if (blocks > 2048) blocks = 2048;
        hipExtLaunchKernelGGL(owner_pad_kernel, dim3(unsigned(blocks)), dim3(kThreads), 0, stream,
                              n_real > 0 ? nullptr : ev.start, ev.stop, 0, a.st, n_real);
        const hipError_t e = hipGetLastError();
        if (e != hipSuccess) return e;
    }
    hipLaunchKernelGGL(publish_flag_kernel, dim3(1), dim3(1), 0, stream, a.st.flag, a.st.epoch, a.st.host_word);
    return hipGetLastError();
}

}  // namespace zp
