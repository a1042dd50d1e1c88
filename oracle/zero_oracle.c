/*
 * zero_oracle.c -- plain scalar CPU oracle for one rank's ZeRO-DP shard step.
 *
 * TEST INFRASTRUCTURE ONLY.  This file is the checker, not the product: only
 * the test suite, the smoke entry and the benchmark's CPU-baseline leg load it.
 * It shares no code, header or constant table with the HIP library.
 *
 * Sources (the "ZeRO: Memory Optimizations Toward Training Trillion Parameter
 * Models" explainer page at azimuth.plus, which describes the method):
 *   - model-states paragraph: the model states are
 *     fp16 parameters, fp16 gradients and an fp32 Adam state made of a master
 *     copy of the parameters, a momentum and a variance.  Precision is therefore
 *     fixed by the page: fp16 storage for parameters/gradients, fp32 for the
 *     optimizer state.  Every fp32 operation below rounds once, in the order
 *     written (the file is compiled with -ffp-contract=off, no fast-math).
 *   - Stage 2 (P_os+g) paragraph: a rank receives
 *     only the reduced slice of the gradients for the partition it owns
 *     (reduce-scatter), updates only that partition, and the updated fp16
 *     parameters are then all-gathered.  The local arithmetic of the reduce is
 *     the sum of R fp16 contributions for that slice.
 *   - Stage 1 (P_os) paragraph: each rank
 *     updates only its own partition of the parameters with its partition of
 *     the optimizer state.
 * The pages name Adam but never write the update rule; the rule used here is
 * the textbook Adam of Kingma and Ba (bias-corrected first and second moment,
 * epsilon added outside the square root).  Loss scaling is not on the pages
 * either; the reading used is "unscale by 1/scale, and if any reduced value is
 * not finite, skip the whole step".
 *
 * Nothing here is blocked, fused or vectorised: one element at a time, one
 * operation per rounding.
 */
#include <math.h>
#include <stdint.h>
#include <string.h>

/* ------------------------------------------------------------------------ */
/* IEEE 754 binary16, written from the format's definition:                  */
/*   1 sign bit, 5 exponent bits (bias 15), 10 fraction bits.                */
/*   exponent 0      -> subnormal: value = fraction * 2^-24                  */
/*   exponent 1..30  -> normal:    value = (1024 + fraction) * 2^(exp - 25)  */
/*   exponent 31     -> fraction 0: infinity, otherwise NaN                  */
/* ------------------------------------------------------------------------ */

float zo_half_to_float(uint16_t h)
{
    int sign = (h >> 15) & 1;
    int expo = (h >> 10) & 0x1F;
    int frac = h & 0x3FF;
    float mag;
    if (expo == 0) {
        mag = ldexpf((float)frac, -24);          /* exact: frac < 2^10 */
    } else if (expo == 31) {
        mag = (frac == 0) ? INFINITY : NAN;
    } else {
        mag = ldexpf((float)(1024 + frac), expo - 25);   /* exact: < 2^11 */
    }
    return sign ? -mag : mag;
}

/* Round an fp32 value to the nearest binary16 value, ties to even.
 *
 * For a finite magnitude a, the spacing of binary16 values around a is
 * q = 2^-24 below 2^-14 (the subnormal range) and q = 2^(floor(log2 a) - 10)
 * above.  n = a / q is then an exact scaling; round n to an integer with ties
 * to even and the rounded magnitude is n * q.  A result of 2^16 or more does
 * not fit (the largest finite value is 65504) and becomes infinity.
 */
uint16_t zo_float_to_half(float x)
{
    uint16_t sign = signbit(x) ? 0x8000 : 0;
    float a = fabsf(x);
    if (isnan(x))
        return (uint16_t)(sign | 0x7E00);
    if (isinf(a))
        return (uint16_t)(sign | 0x7C00);
    if (a == 0.0f)
        return sign;

    int e2;                       /* a = f * 2^e2 with f in [0.5, 1) */
    (void)frexpf(a, &e2);
    int floor_log2 = e2 - 1;      /* a in [2^floor_log2, 2^(floor_log2+1)) */
    int qexp = (floor_log2 < -14) ? -24 : floor_log2 - 10;

    float n = ldexpf(a, -qexp);   /* exact power-of-two scaling */
    float whole = floorf(n);
    float frac = n - whole;       /* exact: n has at most 24 significant bits */
    if (frac > 0.5f) {
        whole = whole + 1.0f;
    } else if (frac == 0.5f) {
        if (fmodf(whole, 2.0f) != 0.0f)
            whole = whole + 1.0f;
    }
    /* whole is an integer < 2^12; rounded magnitude is whole * 2^qexp */
    if (whole == 0.0f)
        return sign;
    double r = ldexp((double)whole, qexp);
    if (r >= 65536.0)
        return (uint16_t)(sign | 0x7C00);

    /* encode r */
    if (r < ldexp(1.0, -14)) {
        /* subnormal: r = fraction * 2^-24 */
        uint16_t fr = (uint16_t)ldexp(r, 24);
        return (uint16_t)(sign | fr);
    }
    int re2;
    (void)frexp(r, &re2);
    int rlog2 = re2 - 1;                              /* r in [2^rlog2, 2^(rlog2+1)) */
    uint16_t biased = (uint16_t)(rlog2 + 15);
    uint16_t fr = (uint16_t)(ldexp(r, 10 - rlog2) - 1024.0);  /* exact */
    return (uint16_t)(sign | (biased << 10) | fr);
}

/* Bulk helpers so the Python side can test the conversions on large arrays. */
void zo_half_to_float_n(const uint16_t* in, float* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zo_half_to_float(in[i]);
}

void zo_float_to_half_n(const float* in, uint16_t* out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        out[i] = zo_float_to_half(in[i]);
}

/* ------------------------------------------------------------------------ */
/* Reduce of R contributions (local arithmetic of reduce-scatter).           */
/* The contributions are summed in fp32, contribution 0 first, then 1, ...   */
/* ------------------------------------------------------------------------ */

static float reduce_one(const uint16_t* const* contrib, int32_t R, int64_t i)
{
    float sum = zo_half_to_float(contrib[0][i]);
    for (int32_t r = 1; r < R; ++r)
        sum = sum + zo_half_to_float(contrib[r][i]);
    return sum;
}

/* Writes the R-way fp32 sums (used to test the reduce on its own). */
void zo_reduce(const uint16_t* const* contrib, int32_t R, float* sum_out, int64_t n)
{
    for (int64_t i = 0; i < n; ++i)
        sum_out[i] = reduce_one(contrib, R, i);
}

/* Overflow flag: 1 if any reduced value over the n elements is not finite. */
int32_t zo_overflow_flag(const uint16_t* const* contrib, int32_t R, int64_t n)
{
    int32_t flag = 0;
    for (int64_t i = 0; i < n; ++i) {
        float s = reduce_one(contrib, R, i);
        if (!isfinite(s))
            flag = 1;
    }
    return flag;
}

/* ------------------------------------------------------------------------ */
/* Mixed-precision Adam on the owned partition (textbook Kingma-Ba form).    */
/*                                                                          */
/* Called only for a step that is taken (no overflow); t is the step number */
/* after this step (1 for the first step).  For each element i:             */
/*   g     = (sum of the R contributions) * (1 / scale)                     */
/*   g     = g + wd * p                  (only when wd != 0)                */
/*   m     = beta1 * m + (1 - beta1) * g                                    */
/*   v     = beta2 * v + (1 - beta2) * g * g                                */
/*   mhat  = m / (1 - beta1^t)                                              */
/*   vhat  = v / (1 - beta2^t)                                              */
/*   p     = p - lr * (mhat / (sqrt(vhat) + eps))                           */
/*   out16 = p rounded to binary16 (nearest, ties to even)                  */
/* The bias-correction factors 1 - beta^t are formed in double from the     */
/* float betas and rounded once to float.                                   */
/* ------------------------------------------------------------------------ */

void zo_adam_apply(const uint16_t* const* contrib, int32_t R,
                   float* p, float* m, float* v, uint16_t* out16, int64_t n,
                   float scale, int64_t t,
                   float lr, float beta1, float beta2, float eps, float wd)
{
    float inv_scale = 1.0f / scale;
    float one_minus_b1 = 1.0f - beta1;
    float one_minus_b2 = 1.0f - beta2;
    float bc1 = (float)(1.0 - pow((double)beta1, (double)t));
    float bc2 = (float)(1.0 - pow((double)beta2, (double)t));

    for (int64_t i = 0; i < n; ++i) {
        float g = reduce_one(contrib, R, i) * inv_scale;
        if (wd != 0.0f)
            g = g + wd * p[i];
        float mi = beta1 * m[i] + one_minus_b1 * g;
        float vi = beta2 * v[i] + one_minus_b2 * (g * g);
        float mhat = mi / bc1;
        float vhat = vi / bc2;
        float denom = sqrtf(vhat) + eps;
        float pi = p[i] - lr * (mhat / denom);
        m[i] = mi;
        v[i] = vi;
        p[i] = pi;
        if (out16)
            out16[i] = zo_float_to_half(pi);
    }
}
