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

// Per-group quantization constants.
//
// s = fl32(amax / 448), computed as the fp32 rounding of the fp64 product amax * fl64(1/448).  That is the
// correctly rounded quotient: amax is a bf16 value A * 2^e (A < 2^8), so amax / 448 = (A / 7) * 2^(e-6) is
// either exact in fp32 (7 divides A) or a non-dyadic number at relative distance >= 2^-28 from every fp32
// rounding boundary, far more than the fp64 product's error (< 2^-52).
// rcp approximates 1 / s within 1 ulp (hardware reciprocal); the exact path forms its quotient as
// (x * p2) * r with p2 a power of two that keeps the reciprocal finite for tiny s (both products by p2
// are exact).
struct GroupScale {
    float s;     // stored scale
    float r;     // ~1 / (s * p2) (1 ulp), +inf when s == 0
    float p2;    // 2^64 when s < 2^-64, else 1
    float rcp;   // ~1 / s (1 ulp), used by the fast path
    bool tiny;   // s < 2^-64 (including the all-zero group): every element takes the exact path
};

__device__ __forceinline__ GroupScale make_group_scale(float amax) {
    GroupScale g;
    g.s = (float)((double)amax * (1.0 / 448.0));
    g.tiny = !(g.s >= 0x1p-64f);
    g.p2 = g.tiny ? 0x1p64f : 1.0f;
    g.r = __builtin_amdgcn_rcpf(g.s * g.p2);
    g.rcp = __builtin_amdgcn_rcpf(g.s);
    return g;
}

// Maximum over the 16 lanes of a DPP row (lanes 16k .. 16k+15), without LDS traffic: swap within pairs,
// within quads, mirror within each half row, mirror the row.
__device__ __forceinline__ float row16_max(float a) {
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0xB1, 0xF, 0xF, false)));
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x4E, 0xF, 0xF, false)));
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x141, 0xF, 0xF, false)));
    a = fmaxf(a, __int_as_float(__builtin_amdgcn_update_dpp(0, __float_as_int(a), 0x140, 0xF, 0xF, false)));
    return a;
}

// Magnitudes of two bf16 values packed in a word (sign bits cleared), and the lane-wise maximum of two such
// words.  For finite values the order of the 15 magnitude bits is the order of the magnitudes, so maxima are
// taken on 16-bit integers, two per instruction.
typedef unsigned short u16x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t mag2(uint32_t w) { return w & 0x7FFF7FFFu; }
__device__ __forceinline__ uint32_t pkmax16(uint32_t a, uint32_t b) {
    return __builtin_bit_cast(uint32_t, __builtin_elementwise_max(__builtin_bit_cast(u16x2_t, a),
                                                                  __builtin_bit_cast(u16x2_t, b)));
}
__device__ __forceinline__ uint32_t max_mag2(uint32_t a, uint32_t b) { return pkmax16(mag2(a), mag2(b)); }

// Largest magnitude among the eight bf16 values of v, as a bf16 bit pattern.
__device__ __forceinline__ uint32_t amax8_bits(const uint4& v) {
    const uint32_t m = pkmax16(max_mag2(v.x, v.y), max_mag2(v.z, v.w));
    return max(m & 0xFFFFu, m >> 16);
}

// Integer maximum over the 16 lanes of a DPP row (same exchange pattern as row16_max; 0 is the identity).
__device__ __forceinline__ uint32_t row16_max_u32(uint32_t a) {
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0xB1, 0xF, 0xF, false));
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x4E, 0xF, 0xF, false));
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x141, 0xF, 0xF, false));
    a = max(a, (uint32_t)__builtin_amdgcn_update_dpp(0, (int)a, 0x140, 0xF, 0xF, false));
    return a;
}

// Approximate quotient x / s (relative error <= 2^-23 + 2^-48): exact +-0 for an all-zero group.
__device__ __forceinline__ float approx_quotient(float x, const GroupScale& g) {
    return (g.s == 0.0f) ? x : (x * g.p2) * g.r;
}

// Exact rounding near a midpoint.  `q` approximates x / s within 3 ulps and `m` is the E4M3 rounding
// midpoint nearest to it (see encode8).  The side of m on which the exact quotient lies is the sign of
// |x| p2 - m (s p2), formed by one fused multiply-add: m has at most 5 significant bits and both products by
// the power of two p2 are exact, so the fma rounds the exact difference once, which keeps its sign.  Both
// terms are multiples of 2^-133 (|x| p2 because x is bf16; m s p2 because m is a multiple of 2^-10 and s p2 a
// normal fp32 >= 2^-85), so a nonzero difference is at least 2^-133 and never rounds to zero.  The result
// is m's fp32 neighbour on that side, which the hardware conversion rounds away from m, or m itself on an
// exact tie, which the conversion rounds to the even code.
__device__ __forceinline__ float resolve_at_midpoint(float x, float m, const GroupScale& g) {
    const float d = fmaf(-m, g.s * g.p2, fabsf(x) * g.p2);
    const uint32_t mb = __float_as_uint(m);
    const float r = d > 0.0f ? __uint_as_float(mb + 1u) : (d < 0.0f ? __uint_as_float(mb - 1u) : m);
    return copysignf(r, x);
}

// Two E4M3 codes packed into the low (HI_WORD=false) or high 16 bits of `old`.  The quotients never
// exceed 448.9 (< 464, the first value the conversion would not round to 448), so no clamp is needed.
template <bool HI_WORD>
__device__ __forceinline__ uint32_t cvt2_e4m3(float a, float b, uint32_t old) {
    return (uint32_t)__builtin_amdgcn_cvt_pk_fp8_f32(a, b, (int)old, HI_WORD);
}

// Eight codes of one group, packed little-endian into two uint32.
//
// q = fl32(x * rcp) is within 3 ulps of x / s (rcp within 1 ulp of 1 / s, one more rounding; a tiny scale
// uses the p2-scaled quotient, same bound), and the hardware conversion rounds q to nearest even.  That
// equals the rounding of the exact quotient unless an E4M3 rounding midpoint lies between q and x / s, or q
// is itself one: such a midpoint is within 3 ulps of q.  Each element is screened on its own:
//   - normal range (>= 2^-6): the midpoints are 1.mmm1 x 2^E, patterns that are odd multiples of 2^19 (low
//     20 bits exactly 0x80000), at least 2^(E-4) inside their binade; a q within 3 ulps shares the binade,
//     so its pattern is within 3 of the midpoint's.  Screen: low 20 bits of (pattern + 4 - 0x80000) <= 8;
//     the midpoint is then the pattern rounded to a multiple of 2^19.
//   - below 2^-6 the midpoints are the odd multiples of 2^-10: every nonzero q at or below 2^-6 + 3 ulps is
//     screened, with the midpoint (floor(512 |q|) + 1/2) / 512 of its quantum cell.
// The representable values (low 20 bits zero), among them the 448 of each group's largest element, pass.
// A screened element (about 0.5 % of LLM-like bf16 data, where x and amax share 8-bit significands) takes
// resolve_at_midpoint in a branch of its own, so a wave pays for the element positions its lanes flagged.
__device__ __forceinline__ uint2 pack8(const float q[8]) {
    // the low-half conversions write into the register of their second operand (its old bits are replaced
    // by the high-half conversion), so no register has to be cleared first
    uint2 out;
    out.x = cvt2_e4m3<true>(q[2], q[3], cvt2_e4m3<false>(q[0], q[1], __float_as_uint(q[1])));
    out.y = cvt2_e4m3<true>(q[6], q[7], cvt2_e4m3<false>(q[4], q[5], __float_as_uint(q[5])));
    return out;
}

// Midpoint of the E4M3 quantum cell that holds |q| (see encode8): q's pattern rounded to a multiple of 2^19 in
// the normal range, (floor(512 |q|) + 1/2) / 512 below 2^-6.
__device__ __forceinline__ float cell_midpoint(float q, bool small) {
    const float aq = fabsf(q);
    return small ? (floorf(aq * 512.0f) + 0.5f) * 0x1p-9f
                 : __uint_as_float((__float_as_uint(aq) + 0x40000u) & 0xFFF80000u);
}

__device__ __forceinline__ uint2 encode8(const float x[8], const GroupScale& g) {
    constexpr uint32_t kSmall = 2u * (0x3C800000u + 3u) - 2u;    // (2 |q| pattern - 2) <= kSmall: 0 < |q| <= 2^-6 + 3 ulps
    float q[8];
    uint32_t smin = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        q[i] = x[i] * g.rcp;
        smin = min(smin, (__float_as_uint(q[i]) << 1) - 2u);    // +-0 wraps to the top
    }
    if (g.tiny) {
#pragma unroll
        for (int i = 0; i < 8; ++i) q[i] = approx_quotient(x[i], g);
        smin = 0;     // screen every element below
    }
    // (pattern + 4 - 0x80000) << 12 with the constant held in a scalar register, so that each element's screen
    // is one v_add_lshl_u32 (the compiler would otherwise rematerialize the literal into a vector register)
    uint32_t k_mid;
    asm("s_mov_b32 %0, 0xfff80004" : "=s"(k_mid));
    if (smin <= kSmall) {
        // rare: some quotient of this lane is at or below 2^-6 (or the scale is tiny)
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            const uint32_t b = __float_as_uint(q[i]);
            const bool small = (b << 1) - 2u <= kSmall;
            if (small || ((b + k_mid) << 12) <= (8u << 12)) q[i] = resolve_at_midpoint(x[i], cell_midpoint(q[i], small), g);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            if (((__float_as_uint(q[i]) + k_mid) << 12) <= (8u << 12))
                q[i] = resolve_at_midpoint(x[i], cell_midpoint(q[i], false), g);
        }
    }
    return pack8(q);
}

}  // namespace jetfp8
