// vec16.hpp -- device helpers for 16-byte vectors of eight fp16 bit patterns
// shared by the pack and reduce-to-owner kernels.
#pragma once

#include <hip/hip_runtime.h>

#include <cstdint>

namespace zp {

typedef uint32_t u32x4 __attribute__((ext_vector_type(4)));

// fp16 bit pattern -> fp32 (exact) and fp32 -> fp16 bit pattern (round to
// nearest even, subnormals kept; the hardware conversions under the default
// rounding and denormal modes).
__device__ __forceinline__ float h2f(uint32_t bits) {
    return float(__builtin_bit_cast(_Float16, uint16_t(bits)));
}

__device__ __forceinline__ uint32_t f2h(float x) {
    return uint32_t(__builtin_bit_cast(uint16_t, _Float16(x)));
}

__device__ __forceinline__ uint32_t funnel16(uint32_t lo, uint32_t hi) {
    return (lo >> 16) | (hi << 16);
}

// Elements ph .. ph+7 of the 16 elements held in a (0..7) and b (8..15).
__device__ __forceinline__ u32x4 window8(u32x4 a, u32x4 b, int ph) {
    const uint32_t w0 = a.x, w1 = a.y, w2 = a.z, w3 = a.w;
    const uint32_t w4 = b.x, w5 = b.y, w6 = b.z, w7 = b.w;
    switch (ph) {
        case 0: return a;
        case 1: return u32x4{funnel16(w0, w1), funnel16(w1, w2), funnel16(w2, w3), funnel16(w3, w4)};
        case 2: return u32x4{w1, w2, w3, w4};
        case 3: return u32x4{funnel16(w1, w2), funnel16(w2, w3), funnel16(w3, w4), funnel16(w4, w5)};
        case 4: return u32x4{w2, w3, w4, w5};
        case 5: return u32x4{funnel16(w2, w3), funnel16(w3, w4), funnel16(w4, w5), funnel16(w5, w6)};
        case 6: return u32x4{w3, w4, w5, w6};
        default: return u32x4{funnel16(w3, w4), funnel16(w4, w5), funnel16(w5, w6), funnel16(w6, w7)};
    }
}

// Eight consecutive fp16 patterns starting at p, read as aligned 16-byte
// blocks only when those blocks lie inside [lo, hi) (the tensor holding p);
// otherwise element by element.  Requires [p, p + 8) inside [lo, hi).
__device__ __forceinline__ u32x4 load8(const uint16_t* p, const uint16_t* lo, const uint16_t* hi) {
    const int ph = int((reinterpret_cast<uintptr_t>(p) & 15) >> 1);
    const uint16_t* base = p - ph;
    if (ph == 0) return *reinterpret_cast<const u32x4*>(p);
    if (base >= lo && base + 16 <= hi) {
        const u32x4 a = *reinterpret_cast<const u32x4*>(base);
        const u32x4 b = *reinterpret_cast<const u32x4*>(base + 8);
        return window8(a, b, ph);
    }
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = uint32_t(p[2 * d]) | (uint32_t(p[2 * d + 1]) << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace zp
