// Block-scaled FP8 GEMM for gfx950 (CDNA4): one "NT" core for the forward, DGrad and WGrad GEMMs of the
// Jet-RL unified FP8 flow (Jet-RL explainers, "Schema de Quantification": FP8 GEMMs with 1x128 activation
// groups and 128x128 weight blocks; DGrad / WGrad in FP8 with 1x128 and 128x1 groupings).
//
//   C[i][j] = sum_g  As[g][i] * sb(j, g) * sum_{k in g} A[i][k] * B[j][k]      (A, B contiguous along k)
//
// One quantization group (128 along k) is exactly one V_MFMA_F32_16X16X128_F8F6F4 per 16x16 output tile,
// issued with a zero accumulator; its fp32 result is promoted into the fp32 accumulator with
// acc = fma(p, fl32(sa * sb), acc), groups in ascending order.  The per-element operation sequence does
// not depend on the tile an element lands in, so a row's bits do not depend on M.
#include "jetfp8_common.h"
#include "jetfp8_launch.h"

namespace jetfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));

// 16x16x128 FP8 (E4M3 x E4M3) matrix product with C = 0.  Lane l supplies row (l % 16) of A and of B,
// bytes k = 32 * (l / 16) .. +31; the result element v of lane l is D[4 * (l / 16) + v][l % 16].
__device__ __forceinline__ v4f mfma_group(const v8i& a, const v8i& b) {
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

constexpr int BM = 128, BN = 128, BK = 128;  // BK = one quantization group

// LDS tile layout: 128 rows x 128 bytes; the 16-byte chunk c of row r is stored at chunk c ^ (r & 7).
__device__ __forceinline__ int swz(int r, int c) { return r * BK + ((c ^ (r & 7)) << 4); }

template <bool ROW_SCALED_B>
__global__ __launch_bounds__(256) void gemm_nt_kernel(const uint8_t* __restrict__ A, const float* __restrict__ As,
                                                      const uint8_t* __restrict__ B, const float* __restrict__ Bs,
                                                      uint16_t* __restrict__ Cout, int64_t I, int64_t J, int64_t Kc,
                                                      int64_t sbj, int64_t sbg) {
    __shared__ __attribute__((aligned(16))) uint8_t lds_a[BM * BK];
    __shared__ __attribute__((aligned(16))) uint8_t lds_b[BN * BK];
    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    const int64_t i0 = (int64_t)blockIdx.y * BM, j0 = (int64_t)blockIdx.x * BN;
    const int G = (int)(Kc / BK);

    // Global -> register staging: 4 x 16 bytes of A and of B per thread (rows (t >> 3) + 32c, chunk t & 7).
    // Rows of A past I re-read row I - 1 (always in bounds); an output row depends only on its own A row
    // and rows past I are never stored, so their contents do not matter.
    const int srow = t >> 3, schk = t & 7;
    auto arow = [&](int c) -> int64_t { const int64_t r = i0 + srow + 32 * c; return r < I ? r : I - 1; };
    const uint8_t* const pa0 = A + arow(0) * Kc + schk * 16;
    const uint8_t* const pa1 = A + arow(1) * Kc + schk * 16;
    const uint8_t* const pa2 = A + arow(2) * Kc + schk * 16;
    const uint8_t* const pa3 = A + arow(3) * Kc + schk * 16;
    const uint8_t* const pb0 = B + (j0 + srow) * Kc + schk * 16;
    const int64_t bstep = 32 * Kc;
    uint4 ra0, ra1, ra2, ra3, rb0, rb1, rb2, rb3;
#define JETFP8_GLOAD(g)                                                                        \
    {                                                                                          \
        const int64_t go = (int64_t)(g) * BK;                                                  \
        ra0 = *reinterpret_cast<const uint4*>(pa0 + go);                                       \
        ra1 = *reinterpret_cast<const uint4*>(pa1 + go);                                       \
        ra2 = *reinterpret_cast<const uint4*>(pa2 + go);                                       \
        ra3 = *reinterpret_cast<const uint4*>(pa3 + go);                                       \
        rb0 = *reinterpret_cast<const uint4*>(pb0 + go);                                       \
        rb1 = *reinterpret_cast<const uint4*>(pb0 + bstep + go);                               \
        rb2 = *reinterpret_cast<const uint4*>(pb0 + 2 * bstep + go);                           \
        rb3 = *reinterpret_cast<const uint4*>(pb0 + 3 * bstep + go);                           \
    }
#define JETFP8_SSTORE()                                                                        \
    {                                                                                          \
        *reinterpret_cast<uint4*>(lds_a + swz(srow, schk)) = ra0;                              \
        *reinterpret_cast<uint4*>(lds_a + swz(srow + 32, schk)) = ra1;                         \
        *reinterpret_cast<uint4*>(lds_a + swz(srow + 64, schk)) = ra2;                         \
        *reinterpret_cast<uint4*>(lds_a + swz(srow + 96, schk)) = ra3;                         \
        *reinterpret_cast<uint4*>(lds_b + swz(srow, schk)) = rb0;                              \
        *reinterpret_cast<uint4*>(lds_b + swz(srow + 32, schk)) = rb1;                         \
        *reinterpret_cast<uint4*>(lds_b + swz(srow + 64, schk)) = rb2;                         \
        *reinterpret_cast<uint4*>(lds_b + swz(srow + 96, schk)) = rb3;                         \
    }

    v4f acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    const int qrow = 4 * (lane >> 4);   // first output row of this lane inside a 16x16 tile
    const int qcol = lane & 15;         // output column of this lane inside a 16x16 tile
    JETFP8_GLOAD(0)
    for (int g = 0; g < G; ++g) {
        __syncthreads();
        JETFP8_SSTORE()
        __syncthreads();
        if (g + 1 < G) { JETFP8_GLOAD(g + 1) }

        // scales of this group
        float sa[4][4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t r = i0 + wm * 64 + tm * 16 + qrow + v;
                sa[tm][v] = As[(int64_t)g * I + (r < I ? r : I - 1)];
            }
        float sb[4];
        if (ROW_SCALED_B) {
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) sb[tn] = Bs[(int64_t)g * J + j0 + wn * 64 + tn * 16 + qcol];
        } else {
            const float v = Bs[(j0 / 128) * sbj + (int64_t)g * sbg];
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) sb[tn] = v;
        }

        // fragments: 32 contiguous bytes (two 16-byte chunks) of one row per lane
        v8i af[4], bfr[4];
        const int cpair = 2 * (lane >> 4);
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int r = wm * 64 + tm * 16 + (lane & 15);
            const uint4 lo = *reinterpret_cast<const uint4*>(lds_a + swz(r, cpair));
            const uint4 hi = *reinterpret_cast<const uint4*>(lds_a + swz(r, cpair + 1));
            af[tm] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int r = wn * 64 + tn * 16 + (lane & 15);
            const uint4 lo = *reinterpret_cast<const uint4*>(lds_b + swz(r, cpair));
            const uint4 hi = *reinterpret_cast<const uint4*>(lds_b + swz(r, cpair + 1));
            bfr[tn] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        // two row-tiles at a time: 8 independent matrix ops in flight, then their promotions
#pragma unroll
        for (int th = 0; th < 4; th += 2) {
            v4f p[2][4];
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn) p[u][tn] = mfma_group(af[th + u], bfr[tn]);
#pragma unroll
            for (int u = 0; u < 2; ++u)
#pragma unroll
                for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                    for (int v = 0; v < 4; ++v) {
                        const float s = sa[th + u][v] * sb[tn];
                        acc[th + u][tn][v] = fmaf(p[u][tn][v], s, acc[th + u][tn][v]);
                    }
        }
    }

    // epilogue: bf16 round to nearest even
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int tn = 0; tn < 4; ++tn)
#pragma unroll
            for (int v = 0; v < 4; ++v) {
                const int64_t r = i0 + wm * 64 + tm * 16 + qrow + v;
                const int64_t c = j0 + wn * 64 + tn * 16 + qcol;
                if (r < I) Cout[r * J + c] = (uint16_t)f32_to_bf16_rne(acc[tm][tn][v]);
            }
#undef JETFP8_GLOAD
#undef JETFP8_SSTORE
}

hipError_t launch_gemm_block_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                      uint16_t* C, int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg,
                                      hipStream_t st) {
    dim3 grid((unsigned)(J / BN), (unsigned)((I + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_nt_kernel<false>, grid, dim3(256), 0, st, A, As, B, Bs, C, I, J, Kc, sbj, sbg);
    return hipGetLastError();
}

hipError_t launch_gemm_row_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                    uint16_t* C, int64_t I, int64_t J, int64_t Kc, hipStream_t st) {
    dim3 grid((unsigned)(J / BN), (unsigned)((I + BM - 1) / BM));
    hipLaunchKernelGGL(gemm_nt_kernel<true>, grid, dim3(256), 0, st, A, As, B, Bs, C, I, J, Kc, (int64_t)0,
                       (int64_t)0);
    return hipGetLastError();
}

}  // namespace jetfp8
