// Device helpers shared by the gfx950 kernels of libjetfp8 (quantize and GEMM).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jetfp8 {

// bf16 bit pattern -> fp32 (exact).
__device__ __forceinline__ float bf16_to_f32(uint32_t b16) { return __uint_as_float(b16 << 16); }

// fp32 -> bf16 bit pattern, round to nearest even (finite inputs).
__device__ __forceinline__ uint32_t f32_to_bf16_rne(float f) {
    uint32_t u = __float_as_uint(f);
    return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16;
}

// Per-group quantization constants.  s = fl32(amax / 448); the element quotient x / s is formed as
// (x * p2) * fl32(1 / (s * p2)) with p2 a power of two that keeps the reciprocal finite for tiny s
// (both products by p2 are exact).
struct GroupScale {
    float s;   // stored scale
    float r;   // fl32(1 / (s * p2)), +inf when s == 0
    float p2;  // 2^64 when s < 2^-64, else 1
};

__device__ __forceinline__ GroupScale make_group_scale(float amax) {
    GroupScale g;
    g.s = __fdiv_rn(amax, 448.0f);
    g.p2 = (g.s < 0x1p-64f) ? 0x1p64f : 1.0f;
    g.r = __frcp_rn(g.s * g.p2);
    return g;
}

// Approximate quotient x / s (relative error <= 2^-23 + 2^-48): exact +-0 for an all-zero group.
__device__ __forceinline__ float approx_quotient(float x, const GroupScale& g) {
    return (g.s == 0.0f) ? x : (x * g.p2) * g.r;
}

// The E4M3 value nearest to the exact quotient x / s.  `q` is the approximate quotient.  Away from an
// E4M3 rounding midpoint q already rounds like the exact quotient, so q is returned and the hardware
// conversion (round to nearest even) finishes the job.  Within 2^-18 quanta of a midpoint -- a band
// wider than q's error -- the side is decided exactly: |x| is compared with midpoint * s in fp64,
// where the product (<= 5 + 24 significant bits) and the difference's sign are exact.
__device__ __forceinline__ float resolve_midpoint(float x, float q, float s) {
    float aq = fabsf(q);
    int e = __builtin_amdgcn_frexp_expf(aq);            // aq = f * 2^e, f in [0.5, 1)
    int qe = max(e - 1, -6) - 3;                        // log2 of the E4M3 quantum at aq
    float y = __builtin_amdgcn_ldexpf(aq, -qe);         // aq in quanta: [8,16) normal, [0,8) subnormal
    float fl = floorf(y);
    float frac = y - fl;
    if (fabsf(frac - 0.5f) > 0x1p-18f) return q;
    double mid = ((double)fl + 0.5) * __builtin_amdgcn_ldexp((double)1.0, qe);
    double d = fabs((double)x) - mid * (double)s;
    float pick;
    if (d > 0.0) pick = fl + 1.0f;
    else if (d < 0.0) pick = fl;
    else pick = (((int)fl & 1) == 0) ? fl : fl + 1.0f;   // exact tie: even code
    return copysignf(__builtin_amdgcn_ldexpf(pick, qe), x);
}

// Two E4M3 codes packed into the low (HI_WORD=false) or high 16 bits of `old`.  The quotients never
// exceed 448.9 (< 464, the first value the conversion would not round to 448), so no clamp is needed.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI_WORD);
}

__device__ __forceinline__ float quantize_value(float x, const GroupScale& g) {
    float q = approx_quotient(x, g);
    return resolve_midpoint(x, q, g.s);
}

// Four codes of one group packed little-endian into a uint32.
__device__ __forceinline__ uint32_t encode4(float x0, float x1, float x2, float x3, const GroupScale& g) {
    uint32_t w = cvt2_e4m3<false>(quantize_value(x0, g), quantize_value(x1, g), 0u);
    return cvt2_e4m3<true>(quantize_value(x2, g), quantize_value(x3, g), w);
}

}  // namespace jetfp8
