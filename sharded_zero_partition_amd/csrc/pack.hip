// pack.hip -- ragged-tensor bucket pack for gfx950.
//
// The constant-size buffers paragraph of the ZeRO explainer page (ZeRO-R)
// fuses many small gradient tensors into one fixed-size buffer so that the
// collective works on large messages.  Fill k of a bucket of B elements is
// the window [k*B, (k+1)*B) of the tensors laid back to back; past the end of
// the last tensor the bucket holds zeros.  The copy is bitwise.
//
// Design: the bucket is cut into 8-element (16-byte) vectors and each thread
// of a grid-stride loop owns whole vectors, so stores are always aligned
// 128-bit writes and the work is balanced no matter how ragged the tensors
// are.  A thread finds the source tensor of its vector with a binary search
// over a chunk-indexed slice of the (sorted) tensor table.  When the 8
// elements come from one tensor it reads them with one 128-bit load, or two
// aligned 128-bit loads and a funnel shift when the source is misaligned
// (the second load is the neighbour thread's first one, so it hits in
// cache); vectors that straddle tensors, touch a tensor edge or the end of
// the stream are gathered element by element.  No LDS: each wave's loads are
// already contiguous.
#include "zp_internal.hpp"

namespace zp {
namespace {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

constexpr int kPackThreads = 256;

// Index of the source tensor holding flat index g (g < psi).
__device__ __forceinline__ int find_src(const PackSrc* __restrict__ src,
                                        const int32_t* __restrict__ first, int shift,
                                        int64_t g) {
    const int64_t c = g >> shift;
    int lo = first[c];
    int hi = first[c + 1];
    while (lo < hi) {
        const int mid = (lo + hi + 1) >> 1;
        if (src[mid].flat_off <= g)
            lo = mid;
        else
            hi = mid - 1;
    }
    return lo;
}

__device__ __forceinline__ uint32_t funnel16(uint32_t lo, uint32_t hi) {
    return (lo >> 16) | (hi << 16);
}

// Elements ph .. ph+7 of the 16 elements held in a (0..7) and b (8..15).
__device__ __forceinline__ u32x4 window8(u32x4 a, u32x4 b, int ph) {
    const uint32_t w0 = a.x, w1 = a.y, w2 = a.z, w3 = a.w;
    const uint32_t w4 = b.x, w5 = b.y, w6 = b.z, w7 = b.w;
    switch (ph) {
        case 1: return u32x4{funnel16(w0, w1), funnel16(w1, w2), funnel16(w2, w3), funnel16(w3, w4)};
        case 2: return u32x4{w1, w2, w3, w4};
        case 3: return u32x4{funnel16(w1, w2), funnel16(w2, w3), funnel16(w3, w4), funnel16(w4, w5)};
        case 4: return u32x4{w2, w3, w4, w5};
        case 5: return u32x4{funnel16(w2, w3), funnel16(w3, w4), funnel16(w4, w5), funnel16(w5, w6)};
        case 6: return u32x4{w3, w4, w5, w6};
        default: return u32x4{funnel16(w3, w4), funnel16(w4, w5), funnel16(w5, w6), funnel16(w6, w7)};
    }
}

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
            const uint32_t val = src[i].ptr[ge - src[i].flat_off];
            w[e >> 1] |= val << (16 * (e & 1));
        }
    }
    return u32x4{w[0], w[1], w[2], w[3]};
}

__global__ __launch_bounds__(kPackThreads) void pack_kernel(const PackLaunch a) {
    const int64_t n_vec = (a.bucket_elems + 7) >> 3;
    const int64_t stride = int64_t(gridDim.x) * kPackThreads;
    for (int64_t j = int64_t(blockIdx.x) * kPackThreads + threadIdx.x; j < n_vec; j += stride) {
        const int64_t o = j << 3;
        const int64_t g = a.fill_base + o;
        const int64_t left = a.bucket_elems - o;
        const int nvalid = left < 8 ? int(left) : 8;
        u32x4 out = u32x4{0u, 0u, 0u, 0u};
        if (g < a.psi) {
            const int i = find_src(a.src, a.first, a.chunk_shift, g);
            const PackSrc s = a.src[i];
            const int64_t rel = g - s.flat_off;
            if (nvalid == 8 && rel + 8 <= s.len) {
                const uint16_t* p = s.ptr + rel;
                const int ph = int((reinterpret_cast<uintptr_t>(p) & 15) >> 1);
                if (ph == 0) {
                    out = *reinterpret_cast<const u32x4*>(p);
                } else {
                    // both aligned 16-byte blocks must lie inside the tensor
                    const uint16_t* base = p - ph;
                    if (base >= s.ptr && base + 16 <= s.ptr + s.len) {
                        const u32x4 lo = *reinterpret_cast<const u32x4*>(base);
                        const u32x4 hi = *reinterpret_cast<const u32x4*>(base + 8);
                        out = window8(lo, hi, ph);
                    } else {
                        out = gather8(a.src, i, g, 8, a.psi);
                    }
                }
            } else {
                out = gather8(a.src, i, g, nvalid, a.psi);
            }
        }
        if (nvalid == 8) {
            *reinterpret_cast<u32x4*>(a.bucket + o) = out;
        } else {
            const uint32_t w[4] = {out.x, out.y, out.z, out.w};
            for (int e = 0; e < nvalid; ++e)
                a.bucket[o + e] = uint16_t(w[e >> 1] >> (16 * (e & 1)));
        }
    }
}

}  // namespace

hipError_t launch_pack(const PackLaunch& a, int cu_count, hipStream_t stream) {
    const int64_t n_vec = (a.bucket_elems + 7) >> 3;
    int64_t blocks = (n_vec + kPackThreads - 1) / kPackThreads;
    const int64_t cap = int64_t(cu_count > 0 ? cu_count : 256) * blocks_per_cu_pack();
    if (blocks > cap) blocks = cap;
    if (blocks < 1) blocks = 1;
    hipLaunchKernelGGL(pack_kernel, dim3(unsigned(blocks)), dim3(kPackThreads), 0, stream, a);
    return hipGetLastError();
}

}  // namespace zp
