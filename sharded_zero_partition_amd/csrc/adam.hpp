// adam.hpp -- the per-element arithmetic of the shard step, shared by the
// fused step kernel and the owner step (which feeds it from ragged tensors).
//
// Textbook Adam (Kingma and Ba: bias-corrected first and second moments,
// epsilon outside the square root) on the fp32 master, momentum and variance
// of the ZeRO explainer page's model-states paragraph; one rounding per
// operation, in the order written (no contraction, IEEE division and square
// root), so both kernels match a scalar reference bit for bit.
#pragma once

#include "zp_internal.hpp"

namespace zp {

__device__ __forceinline__ bool not_finite(float x) {
    return (__builtin_bit_cast(uint32_t, x) & 0x7F800000u) == 0x7F800000u;
}

__device__ __forceinline__ void adam_element(const StepLaunch& a, float sum, float& p, float& m,
                                             float& v) {
#pragma clang fp contract(off)
    float g = sum * a.inv_scale;
    if (a.weight_decay != 0.0f) g = g + a.weight_decay * p;
    const float mi = a.beta1 * m + a.one_minus_beta1 * g;
    const float vi = a.beta2 * v + a.one_minus_beta2 * (g * g);
    const float mhat = mi / a.bias_corr1;
    const float vhat = vi / a.bias_corr2;
    const float den = __builtin_sqrtf(vhat) + a.eps;
    p = p - a.lr * (mhat / den);
    m = mi;
    v = vi;
}

}  // namespace zp
