// Fused producers of 1x128 FP8 activations for gfx950: RMSNorm -> quantize and SwiGLU -> quantize.
//
// The 1x128 activation quantization is fused with the operator that produces the activation (Jet-RL
// explainers, "Schema de Quantification"), so the bf16 activation is never written and read back: each
// kernel reads its bf16 inputs once and writes E4M3 codes, fp32 group scales and (optionally) the bf16
// activation itself.  The codes and scales are those of the 1x128 quantizer applied to the bf16 activation,
// bit for bit (same scale and rounding helpers).
//
// Numerics (the producers are not spelled out by the pages; plain readings):
//   RMSNorm: r = fp32 nearest to 1 / sqrt(mean(x^2) + eps); y = bf16(fl32(fl32(x * r) * w)).
//            The sum of squares is formed in fp64 (order-free to ~2^-48 relative), then mean, +eps, sqrt
//            and the reciprocal in fp64 (each correctly rounded), then one rounding to fp32.  That is the
//            nearest fp32 unless the exact value lies within ~2^-47 (relative) of an fp32 rounding midpoint.
//   SwiGLU:  h = bf16 nearest to g * u / (1 + exp(-g)), the exact real value (gate = first half of the
//            columns, up = second half).  An fp32 evaluation is within a few ulps; results within 16 fp32
//            ulps of a bf16 rounding midpoint, tiny (< 2^-100) or huge (>= 2^127) results go through fp64,
//            which decides the rounding unless the exact value lies within ~2^-50 of a midpoint.
#include "jetfp8_common.h"
#include "jetfp8_launch.h"

namespace jetfp8 {

namespace {

__device__ __forceinline__ uint4 ld16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ uint32_t word_of(const uint4& v, int i) {
    return i == 0 ? v.x : i == 1 ? v.y : i == 2 ? v.z : v.w;
}
__device__ __forceinline__ float elem_of(const uint4& v, int i) {
    const uint32_t w = word_of(v, i >> 1);
    return bf16_to_f32((i & 1) ? (w >> 16) : (w & 0xFFFFu));
}

// Codes of the 8 bf16 values held by a lane (bit patterns in hv), as the 1x128 quantizer forms them: the
// group's amax from the 16 lanes of the DPP row, then the scale and the codes of the lane's 8 values.
__device__ __forceinline__ uint2 quantize_lane8(const uint4& hv, float& scale) {
    float f[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) f[i] = elem_of(hv, i);
    const GroupScale gs = make_group_scale(bf16_to_f32(row16_max_u32(amax8_bits(hv))));
    scale = gs.s;
    return encode8(f, gs);
}

// Wave-wide sum of a double (xor butterfly over the 64 lanes; every lane ends with the total).
__device__ __forceinline__ double wave_sum(double v) {
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) v += __shfl_xor(v, m, 64);
    return v;
}

// fp32 bit pattern of v rounded to odd: the nearest fp32 toward zero, with its last bit set when that is
// not v itself.  Rounding this pattern to bf16 (16 bits shorter) to nearest even gives the correct rounding
// of v; |v| beyond the fp32 range becomes the largest fp32 with the sticky bit (so bf16 gives infinity).
__device__ __forceinline__ uint32_t f64_to_f32_odd_bits(double v) {
    const float f = (float)v;
    uint32_t b = __float_as_uint(f);
    const double av = fabs(v);
    if (fabs((double)f) > av) b -= 1u;                       // step toward zero (|f| > |v| >= 0, so |f| > 0)
    if (fabs((double)__uint_as_float(b)) != av) b |= 1u;
    return b;
}

__device__ __forceinline__ uint32_t f32_bits_to_bf16_rne(uint32_t u) { return (u + 0x7FFFu + ((u >> 16) & 1u)) >> 16; }

// Two fp32 values rounded to bf16, nearest even, packed low / high: one V_CVT_PK_BF16_F32.  It equals
// f32_bits_to_bf16_rne on every finite fp32 pattern (all 2^32 - 2^24 of them compared on gfx950, with the
// library's denormal mode).
typedef __bf16 bf16x2_t __attribute__((ext_vector_type(2)));
typedef float f32x2_t __attribute__((ext_vector_type(2)));
__device__ __forceinline__ uint32_t bf16x2_rne(float a, float b) {
    return __builtin_bit_cast(uint32_t, __builtin_convertvector((f32x2_t){a, b}, bf16x2_t));
}

// exp(-g) for the SwiGLU fast path: 2^t with t = -g log2(e) split as t_hi + t_lo, where t_hi is the fp32
// product and t_lo its rounding error (exact by fma) plus the low part of log2(e); then
// 2^t = 2^t_hi * (1 + t_lo ln 2 + O(t_lo^2)), |t_lo| <= 2^-17.  Relative error: that of the hardware exp2
// plus about one ulp.  Over- and underflow follow 2^t_hi (the callers screen those ranges).
__device__ __forceinline__ float exp_neg(float g) {
    constexpr float kLog2eHi = 1.44269502162933349609375f;      // fl32(log2 e)
    constexpr float kLog2eLo = 1.925963033500011079e-8f;        // log2 e - kLog2eHi
    constexpr float kLn2 = 0.693147180559945309f;
    const float t_hi = -g * kLog2eHi;
    const float t_lo = fmaf(-g, kLog2eHi, -t_hi) + (-g) * kLog2eLo;
    return __builtin_amdgcn_exp2f(t_hi) * fmaf(t_lo, kLn2, 1.0f);
}

// The exact-rounding path of SwiGLU: fp64 evaluation (relative error ~2^-50), rounded to bf16 through a
// round-to-odd fp32.  An fp64 value that is exactly a bf16 midpoint comes from a gate at one end of the range,
// where exp(-g) is below fp64 resolution relative to 1 + exp(-g):
//   - a large gate: h = g u / (1 + exp(-g)) lies just below |g u| in magnitude;
//   - a tiny gate (1 + exp(-g) rounds to 2): h = (g u / 2)(1 + g / 2 + O(g^2)) lies just above |g u / 2| in
//     magnitude for g > 0 and just below for g < 0.
// The midpoint is then stepped by one fp32 ulp to the side of the exact value.
__device__ __noinline__ uint32_t swiglu_bf16_exact(float g, float u) {
    const double gd = g, ud = u;
    const double hd = gd / (1.0 + exp(-gd)) * ud;
    uint32_t b = f64_to_f32_odd_bits(hd);
    if ((b & 0xFFFFu) == 0x8000u) b = (g > 0.0f && g < 1.0f) ? b + 1u : b - 1u;
    return f32_bits_to_bf16_rne(b);
}

// silu(g) * u from the fast fp32 evaluation (rounded to bf16 by the caller), and whether the bf16 value must
// instead be taken from swiglu_bf16_exact (the fast one is then not used).
__device__ __forceinline__ float swiglu_fast(float g, float u, bool& exact) {
    const float sil = g * __builtin_amdgcn_rcpf(1.0f + exp_neg(g));
    const float h = sil * u;
    const uint32_t hb = __float_as_uint(h) & 0x7FFFFFFFu;
    // Exact path for: g < -87 (1 + exp(-g) > 2^125.5: the reciprocal nears the subnormal range); h outside
    // [2^-120, 2^127) (0x03800000, 0x7F000000: fp32 subnormal products, overflow); low 16 bits of h within 6 of
    // 0x8000, i.e. within 6 fp32 ulps of a bf16 rounding midpoint.  For every finite bf16 gate >= -87 the fast
    // silu(g) is within 3.23 * 2^-24 (relative) of the exact value (measured over all of them; for tiny gates
    // it is g / 2, exact to far below that), so the fast h is within 4.3 ulps of silu(g) u, inside the window.
    // (A 16-ulp window sent about 3 times as many elements to the fp64 path: SwiGLU 266 -> 249 us at
    // 16384 x 14336 with 6 ulps; the exhaustive gate x up-significand test passes with either.)
    exact = (g < -87.0f) | (hb - 0x03800000u >= 0x7F000000u - 0x03800000u) | (((hb - 0x7FFAu) & 0xFFFFu) <= 0xCu);
    return h;
}

}  // namespace

// ---------------------------------------------------------------------------------------------------------
// RMSNorm -> 1x128.  A block of 8 waves owns 8 / WPR consecutive rows, WPR waves per row.  A wave holds its part of
// the row in registers: its k-th chunk covers columns 512 c .. +511 (c = part * NCH / WPR + k), lane l columns
// 512 c + 8 l .. +7, so the 16 lanes of a DPP row hold one 128-column group.  With WPR = 2 the two halves of the
// sum of squares meet in LDS and are added in a fixed order, so a lane holds half the values and more waves fit
// per SIMD: rows of 4096 48 VGPRs and 8 waves per SIMD (80 capped, 6 waves, with one wave per row), rows of 5120
// 69 VGPRs (128, 4 waves, through the 16-chunk instantiation): measured 52.8 -> 51.5 us at 16384 x 4096 and
// 268.9 -> 242.3 us at 65536 x 5120, bitwise the same codes, scales and rstd.  The group scales of the block's
// rows are staged in LDS and written as runs per group.  (Four rows per wave, with or without the next row's loads
// issued ahead, measured slower than one: all blocks loaded, then all computed, in step.)
constexpr int RN_WAVES = 8;

template <int NCH, int WPR>
__global__ __launch_bounds__(RN_WAVES * 64) void rmsnorm_quant_kernel(
    const uint16_t* __restrict__ x, const uint16_t* __restrict__ w, int64_t R, int64_t C, float eps,
    uint8_t* __restrict__ q, float* __restrict__ s, float* __restrict__ rstd, uint16_t* __restrict__ y) {
    constexpr int ROWS = RN_WAVES / WPR, HCH = NCH / WPR;
    __shared__ float sc[NCH * 4][ROWS];
    __shared__ double pss[ROWS][WPR];
    const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, lane16 = lane & 15, gl = lane >> 4;
    const int64_t r0 = (int64_t)blockIdx.x * ROWS;
    const double eps_d = (double)eps;
    const int rr = wave / WPR, part = wave % WPR;
    const int64_t row = r0 + rr;
    const bool live = row < R;                                   // wave-uniform
    const int64_t rowc = live ? row : 0;                         // in-bounds stand-in row (nothing stored)
    uint4 v[HCH];
#pragma unroll
    for (int k = 0; k < HCH; ++k) {
        const int64_t col = (int64_t)(part * HCH + k) * 512 + lane * 8;
        v[k] = ld16(x + rowc * C + (col < C ? col : 0));         // in-bounds stand-in past C: not used
    }
    double pa[8] = {0, 0, 0, 0, 0, 0, 0, 0};
#pragma unroll
    for (int k = 0; k < HCH; ++k) {
        if ((int64_t)(part * HCH + k) * 512 + lane * 8 < C) {
#pragma unroll
            for (int i = 0; i < 8; ++i) {
                const double f = (double)elem_of(v[k], i);
                pa[i] = fma(f, f, pa[i]);
            }
        }
    }
    double ss = wave_sum(((pa[0] + pa[1]) + (pa[2] + pa[3])) + ((pa[4] + pa[5]) + (pa[6] + pa[7])));
    if (WPR > 1) {
        if (lane == 0) pss[rr][part] = ss;
        __syncthreads();
        ss = pss[rr][0] + pss[rr][1];
    }
    const float r = (float)(1.0 / sqrt(ss / (double)C + eps_d));
    if (live) {
        if (rstd && lane == 0 && part == 0) rstd[row] = r;
#pragma unroll
        for (int k = 0; k < HCH; ++k) {
            const int c = part * HCH + k;
            const int64_t col = (int64_t)c * 512 + lane * 8;
            if (c * 512 >= C) break;                              // whole chunk past the row (uniform)
            const bool ok = col < C;
            const uint4 wv = ld16(w + (ok ? col : 0));
            uint32_t hw[4];
#pragma unroll
            for (int kk = 0; kk < 4; ++kk) {
                const float y0 = (elem_of(v[k], 2 * kk) * r) * elem_of(wv, 2 * kk);
                const float y1 = (elem_of(v[k], 2 * kk + 1) * r) * elem_of(wv, 2 * kk + 1);
                hw[kk] = bf16x2_rne(y0, y1);
            }
            const uint4 yv = make_uint4(hw[0], hw[1], hw[2], hw[3]);
            float scale;
            const uint2 codes = quantize_lane8(yv, scale);
            if (ok) {
                *reinterpret_cast<uint2*>(q + row * C + col) = codes;
                if (y) *reinterpret_cast<uint4*>(y + row * C + col) = yv;
                if (lane16 == 0) sc[c * 4 + gl][rr] = scale;
            }
        }
    }
    __syncthreads();
    const int G = (int)(C / 128);
    for (int i = t; i < G * ROWS; i += RN_WAVES * 64) {
        const int g = i / ROWS, rq = i % ROWS;
        if (r0 + rq < R) s[(int64_t)g * R + r0 + rq] = sc[g][rq];
    }
}

// ---------------------------------------------------------------------------------------------------------
// SwiGLU -> 1x128.  gate_up [R][2F] -> codes [R][F], scales [F/128][R], optional h [R][F].  A block of 8 waves
// owns 32 rows x 512 output columns (4 groups per row); lane l of a wave covers output columns
// c0 + 8 l .. +7 of one row per pass, reading the matching 16 bytes of gate and of up.  All loads of a thread
// are issued first.  Loads and stores go through range-checked buffer descriptors over the block's rows with
// 32-bit lane offsets: rows past R read as zero and their stores are dropped (lanes past the last column store
// nothing).  Clamped 64-bit addresses cost about 12 vector instructions per load: measured 278 -> 259 us at
// 16384 x 14336 and 1858 -> 1812 us at 65536 x 27648, bitwise the same outputs.
constexpr int SG_ROWS = 32, SG_COLS = 512, SG_WAVES = 8, SG_PASSES = SG_ROWS / SG_WAVES;
typedef __amdgpu_buffer_rsrc_t rsrc_sg_t;
typedef unsigned int u32x4_sg __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_sg __attribute__((ext_vector_type(2)));
__device__ __forceinline__ rsrc_sg_t sg_rsrc(const void* base, int bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, bytes, 0x00020000);
}

// Not register-capped: at 64 VGPRs (8 waves per SIMD instead of 7) it spills 3 registers, and the scratch traffic
// adds 10 % to its HBM bytes for a 1 % gain on the bench data.
__global__ __launch_bounds__(SG_WAVES * 64) void swiglu_quant_kernel(const uint16_t* __restrict__ gu, int64_t R,
                                                                      int64_t F, uint8_t* __restrict__ q,
                                                                      float* __restrict__ s, uint16_t* __restrict__ h,
                                                                      uint32_t col_blocks) {
    __shared__ float sc[4][SG_ROWS];
    const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63, gl = lane >> 4, lane16 = lane & 15;
    const uint32_t cb = blockIdx.x % col_blocks, rb = blockIdx.x / col_blocks;
    const int64_t c0 = (int64_t)cb * SG_COLS, r0 = (int64_t)rb * SG_ROWS;
    const int col = (int)c0 + lane * 8;
    const bool col_ok = col < F;                                 // F is a multiple of 128
    const int Fi = (int)F;
    // the block's rows through range-checked descriptors with scalar bases: rows past R read as zero and their
    // stores are dropped; 32-bit lane offsets (the launcher bounds 32 rows of gate_up below 2^31 bytes)
    const int nrows = (int)min((int64_t)SG_ROWS, R - r0);
    const rsrc_sg_t rin = sg_rsrc(gu + r0 * 2 * F, nrows * 4 * Fi);
    const rsrc_sg_t rq = sg_rsrc(q + r0 * F, nrows * Fi);
    const rsrc_sg_t rh = sg_rsrc(h ? h + r0 * F : (uint16_t*)nullptr, h ? nrows * 2 * Fi : 0);
    uint4 gv[SG_PASSES], uv[SG_PASSES];
#pragma unroll
    for (int p = 0; p < SG_PASSES; ++p) {
        // the row offset goes into the lane offset, which the range check covers; the largest lane offset,
        // ro + 2 (F + col) <= 128 F + 1024, stays below 2^31 because the launcher bounds 128 F by 2^31 and F is a
        // multiple of 128 (so 128 F <= 2^31 - 2^14)
        const int ro = (p * SG_WAVES + wave) * 4 * Fi;
        const u32x4_sg a = __builtin_amdgcn_raw_buffer_load_b128(rin, ro + 2 * col, 0, 0);
        const u32x4_sg b = __builtin_amdgcn_raw_buffer_load_b128(rin, ro + 2 * (Fi + col), 0, 0);
        gv[p] = make_uint4(a[0], a[1], a[2], a[3]);
        uv[p] = make_uint4(b[0], b[1], b[2], b[3]);
    }
#pragma unroll
    for (int p = 0; p < SG_PASSES; ++p) {
        // fast values of the lane's 8 elements without branches, rounded to bf16 in pairs, then one rarely taken
        // branch that replaces the flagged ones by the exact path
        float hf[8];
        uint32_t need = 0;
#pragma unroll
        for (int i = 0; i < 8; ++i) {
            bool ex;
            hf[i] = swiglu_fast(elem_of(gv[p], i), elem_of(uv[p], i), ex);
            need |= (uint32_t)ex << i;
        }
        uint32_t hw[4];
#pragma unroll
        for (int k = 0; k < 4; ++k) hw[k] = bf16x2_rne(hf[2 * k], hf[2 * k + 1]);
        if (__builtin_expect(need != 0, 0)) {
            for (int i = 0; i < 8; ++i)
                if ((need >> i) & 1u) {
                    const uint32_t e = swiglu_bf16_exact(elem_of(gv[p], i), elem_of(uv[p], i));
                    hw[i >> 1] = (i & 1) ? ((hw[i >> 1] & 0xFFFFu) | (e << 16)) : ((hw[i >> 1] & 0xFFFF0000u) | e);
                }
        }
        const uint4 hv = make_uint4(hw[0], hw[1], hw[2], hw[3]);
        float scale;
        const uint2 codes = quantize_lane8(hv, scale);
        if (col_ok) {
            const int so = (p * SG_WAVES + wave) * Fi;
            const u32x2_sg cw = {codes.x, codes.y};
            __builtin_amdgcn_raw_buffer_store_b64(cw, rq, so + col, 0, 0);
            if (h) {
                const u32x4_sg hw4 = {hv.x, hv.y, hv.z, hv.w};
                __builtin_amdgcn_raw_buffer_store_b128(hw4, rh, 2 * (so + col), 0, 0);
            }
        }
        if (lane16 == 0) sc[gl][p * SG_WAVES + wave] = scale;
    }
    __syncthreads();
    if (t < 4 * SG_ROWS) {
        const int g = t / SG_ROWS, r = t % SG_ROWS;
        const int64_t gg = c0 / 128 + g;
        if (gg * 128 < F && r0 + r < R) s[gg * R + r0 + r] = sc[g][r];
    }
}

hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* w, int64_t R, int64_t C, float eps, uint8_t* q,
                                float* s, float* rstd, uint16_t* y, hipStream_t st) {
    if (C > kRmsNormMaxCols) return hipErrorInvalidValue;
    const dim3 block(RN_WAVES * 64);
    const dim3 grid1((unsigned)((R + RN_WAVES - 1) / RN_WAVES)), grid2((unsigned)((R + RN_WAVES / 2 - 1) / (RN_WAVES / 2)));
    const int nch = (int)((C + 511) / 512);
    if (nch <= 2) hipLaunchKernelGGL((rmsnorm_quant_kernel<2, 1>), grid1, block, 0, st, x, w, R, C, eps, q, s, rstd, y);
    else if (nch <= 4) hipLaunchKernelGGL((rmsnorm_quant_kernel<4, 1>), grid1, block, 0, st, x, w, R, C, eps, q, s, rstd, y);
    else if (nch <= 8) hipLaunchKernelGGL((rmsnorm_quant_kernel<8, 2>), grid2, block, 0, st, x, w, R, C, eps, q, s, rstd, y);
    else if (nch <= 10) hipLaunchKernelGGL((rmsnorm_quant_kernel<10, 2>), grid2, block, 0, st, x, w, R, C, eps, q, s, rstd, y);
    else if (nch <= 12) hipLaunchKernelGGL((rmsnorm_quant_kernel<12, 2>), grid2, block, 0, st, x, w, R, C, eps, q, s, rstd, y);
    else hipLaunchKernelGGL((rmsnorm_quant_kernel<16, 2>), grid2, block, 0, st, x, w, R, C, eps, q, s, rstd, y);
    return hipGetLastError();
}

bool swiglu_quant_fits(int64_t R, int64_t F) {
    return ((F + SG_COLS - 1) / SG_COLS) * ((R + SG_ROWS - 1) / SG_ROWS) < ((int64_t)1 << 31) &&
           SG_ROWS * 4 * F < ((int64_t)1 << 31);
}

hipError_t launch_swiglu_quant(const uint16_t* gu, int64_t R, int64_t F, uint8_t* q, float* s, uint16_t* h,
                               hipStream_t st) {
    const int64_t col_blocks = (F + SG_COLS - 1) / SG_COLS, row_blocks = (R + SG_ROWS - 1) / SG_ROWS;
    if (!swiglu_quant_fits(R, F)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(swiglu_quant_kernel, dim3((unsigned)(col_blocks * row_blocks)), dim3(SG_WAVES * 64), 0, st,
                       gu, R, F, q, s, h, (uint32_t)col_blocks);
    return hipGetLastError();
}

}  // namespace jetfp8
