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

// Device buffers reached through a table of pointers arrive as generic
// pointers, for which the compiler emits flat loads (address-space check,
// 64-bit VGPR addresses, and a second wait counter shared with LDS and scalar
// loads).  Every buffer here is device global memory, so reads go through
// these global-address-space views instead.
typedef __attribute__((address_space(1))) const u32x4 GlobalU32x4;
typedef __attribute__((address_space(1))) const uint16_t GlobalU16;

__device__ __forceinline__ u32x4 ld16(const uint16_t* p) {    // 16-byte aligned
    return *(const GlobalU32x4*)(p);   // address-space cast
}
__device__ __forceinline__ u32x4 ld16_stream(const uint16_t* p) {   // non-temporal
    return __builtin_nontemporal_load((const GlobalU32x4*)(p));
}
__device__ __forceinline__ uint32_t ld2(const uint16_t* p) {
    return *(const GlobalU16*)(p);
}

// Eight consecutive fp16 patterns starting at p, read as aligned 16-byte
// blocks only when those blocks lie inside [lo, hi) (the tensor holding p);
// otherwise element by element.  Requires [p, p + 8) inside [lo, hi).
__device__ __forceinline__ u32x4 load8(const uint16_t* p, const uint16_t* lo, const uint16_t* hi) {
    const int ph = int((reinterpret_cast<uintptr_t>(p) & 15) >> 1);
    const uint16_t* base = p - ph;
    if (ph == 0) return ld16(p);
    if (base >= lo && base + 16 <= hi) {
        const u32x4 a = ld16(base);
        const u32x4 b = ld16(base + 8);
        return window8(a, b, ph);
    }
    uint32_t w[4];
#pragma unroll
    for (int d = 0; d < 4; ++d) w[d] = ld2(p + 2 * d) | (ld2(p + 2 * d + 1) << 16);
    return u32x4{w[0], w[1], w[2], w[3]};
}

}  // namespace zp
