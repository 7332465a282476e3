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
//
// Layout of the work (large-M kernel):
//   - 512 threads = 8 waves (2 per SIMD), block tile 256 x 128, wave tile 64 x 64 (4 x 4 MFMA tiles);
//   - A and B group tiles stream global -> LDS with global_load_lds_dwordx4 into a double buffer (one
//     barrier per group); LDS rows are 128 bytes with 16-byte chunk c of row r stored at c ^ ((r >> 1) & 7),
//     which makes both the 16-lane fragment reads and the lane-ordered LDS writes bank-conflict free;
//   - block-scaled B (forward, DGrad): s = fl32(sa * sb) is formed once per row and group in LDS, so the
//     VALU does one fma per output per group; row-scaled B (WGrad): the lanes form sa * sb per element;
//   - blocks are renumbered so that each XCD (8 per device, dispatched round robin) works on a compact
//     band of output tiles that share A rows and B rows in its L2.
#include "jetfp8_common.h"
#include "jetfp8_launch.h"

namespace jetfp8 {

typedef int v8i __attribute__((ext_vector_type(8)));
typedef float v4f __attribute__((ext_vector_type(4)));
typedef __attribute__((address_space(3))) void lds_void;

// 16x16x128 FP8 (E4M3 x E4M3) matrix product with C = 0.  Lane l supplies row (l % 16) of A and of B,
// bytes k = 32 * (l / 16) .. +31; the result element v of lane l is D[4 * (l / 16) + v][l % 16].
__device__ __forceinline__ v4f mfma_group(const v8i& a, const v8i& b) {
    const v4f z = {0.0f, 0.0f, 0.0f, 0.0f};
    return __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(a, b, z, 0, 0, 0, 0, 0, 0);
}

constexpr int BK = 128;            // one quantization group along the contraction axis
constexpr int L_BM = 256, L_BN = 128, L_THREADS = 512;
constexpr int L_A_BYTES = L_BM * BK, L_B_BYTES = L_BN * BK;

__device__ __forceinline__ int swz_off(int r, int c) { return r * BK + ((c ^ ((r >> 1) & 7)) << 4); }

// Renumber a 1-D block index so that XCD x (which receives blocks x, x+8, ...) owns a contiguous range of
// tiles, then walk tiles in bands of `group_m` tile-rows, N fastest inside a band.
__device__ __forceinline__ void tile_of_block(int pid, int tiles_m, int tiles_n, int& tm, int& tn) {
    const int T = tiles_m * tiles_n;
    const int per = T / 8, rem = T % 8, xcd = pid % 8, idx = pid / 8;
    const int q = xcd * per + (xcd < rem ? xcd : rem) + idx;
    const int group_m = 8;
    const int band = group_m * tiles_n;
    const int first_m = (q / band) * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int w = q % band;
    tm = first_m + w % gsz;
    tn = w / gsz;
}

template <bool ROW_SCALED_B>
__global__ __launch_bounds__(L_THREADS, 1) void gemm_large_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, uint16_t* __restrict__ Cout, int64_t I, int64_t J, int64_t Kc, int64_t sbj,
    int64_t sbg, int tiles_m, int tiles_n) {
    __shared__ __attribute__((aligned(1024))) uint8_t lds_a[2][L_A_BYTES];
    __shared__ __attribute__((aligned(1024))) uint8_t lds_b[2][L_B_BYTES];
    __shared__ __attribute__((aligned(16))) float lds_s[2][L_BM];      // s (block B) or sa (row B)
    __shared__ __attribute__((aligned(16))) float lds_sb[2][L_BN];     // sb (row B only)

    const int t = threadIdx.x, lane = t & 63, wave = t >> 6;
    const int wm = wave >> 1, wn = wave & 1;
    int tmi, tni;
    tile_of_block(blockIdx.x, tiles_m, tiles_n, tmi, tni);
    const int64_t i0 = (int64_t)tmi * L_BM, j0 = (int64_t)tni * L_BN;
    const int G = (int)(Kc / BK);

    // ---- global -> LDS staging addresses.  Instruction c of wave w fills the 1 KB LDS region
    //      (c * 8 + w), i.e. rows 8 * (c * 8 + w) .. +7; lane l lands at row +l/8, physical chunk l%8.
    const int lrow = lane >> 3, pchunk = lane & 7;
    const uint8_t* ga[4];
#pragma unroll
    for (int c = 0; c < 4; ++c) {
        const int r = (c * 8 + wave) * 8 + lrow;
        const int lc = pchunk ^ ((r >> 1) & 7);
        const int64_t gr = (i0 + r < I) ? i0 + r : I - 1;     // rows past I re-read row I-1, never stored
        ga[c] = A + gr * Kc + lc * 16;
    }
    const uint8_t* gb[2];
#pragma unroll
    for (int c = 0; c < 2; ++c) {
        const int r = (c * 8 + wave) * 8 + lrow;
        const int lc = pchunk ^ ((r >> 1) & 7);
        gb[c] = B + (j0 + r) * Kc + lc * 16;
    }
    auto issue_tiles = [&](int g, int stage) {
        const int64_t go = (int64_t)g * BK;
#pragma unroll
        for (int c = 0; c < 4; ++c)
            __builtin_amdgcn_global_load_lds(ga[c] + go, (lds_void*)(&lds_a[stage][(c * 8 + wave) * 1024]), 16, 0, 0);
#pragma unroll
        for (int c = 0; c < 2; ++c)
            __builtin_amdgcn_global_load_lds(gb[c] + go, (lds_void*)(&lds_b[stage][(c * 8 + wave) * 1024]), 16, 0, 0);
    };

    // ---- scale staging: thread t < 256 owns row i0 + t; for row-scaled B, threads 256..383 own column
    //      j0 + t - 256.  Values for group g + 1 are loaded into registers during group g - 1's compute.
    const int64_t srow = (i0 + (t & 255) < I) ? i0 + (t & 255) : I - 1;
    auto load_scales = [&](int g, float& a, float& b) {
        a = As[(int64_t)g * I + srow];
        if (ROW_SCALED_B) b = (t >= 256 && t < 384) ? Bs[(int64_t)g * J + j0 + (t - 256)] : 0.0f;
        else b = Bs[(j0 / 128) * sbj + (int64_t)g * sbg];
    };
    auto store_scales = [&](int stage, float a, float b) {
        if (ROW_SCALED_B) {
            if (t < 256) lds_s[stage][t] = a;
            else if (t < 384) lds_sb[stage][t - 256] = b;
        } else if (t < 256) {
            lds_s[stage][t] = a * b;                           // s = fl32(sa * sb), once per row and group
        }
    };

    v4f acc[4][4];
#pragma unroll
    for (int a = 0; a < 4; ++a)
#pragma unroll
        for (int b = 0; b < 4; ++b) acc[a][b] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    // prologue: group 0 tiles and scales, group 1 scales in registers
    issue_tiles(0, 0);
    float sa_n, sb_n;
    load_scales(0, sa_n, sb_n);
    store_scales(0, sa_n, sb_n);
    if (G > 1) load_scales(1, sa_n, sb_n);

    const int qrow = 4 * (lane >> 4);      // first output row of this lane inside a 16x16 tile
    const int qcol = lane & 15;            // output column of this lane inside a 16x16 tile
    const int cp = 2 * (lane >> 4);        // logical 16-byte chunk pair of this lane's fragment bytes

    for (int g = 0; g < G; ++g) {
        const int st = g & 1;
        __builtin_amdgcn_s_waitcnt(0);     // this thread's tile loads (and scale loads) have landed
        __syncthreads();                   // ... everyone's; and the other stage is no longer read
        if (g + 1 < G) {
            issue_tiles(g + 1, st ^ 1);
            store_scales(st ^ 1, sa_n, sb_n);
            if (g + 2 < G) load_scales(g + 2, sa_n, sb_n);
        }

        // scales of this lane's 16 rows (and 4 columns for row-scaled B)
        v4f s4[4];
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) s4[tm] = *reinterpret_cast<const v4f*>(&lds_s[st][wm * 64 + tm * 16 + qrow]);
        float sbc[4];
        if (ROW_SCALED_B) {
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) sbc[tn] = lds_sb[st][wn * 64 + tn * 16 + qcol];
        }

        v8i bfr[4];
#pragma unroll
        for (int tn = 0; tn < 4; ++tn) {
            const int r = wn * 64 + tn * 16 + (lane & 15);
            const uint4 lo = *reinterpret_cast<const uint4*>(&lds_b[st][swz_off(r, cp)]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&lds_b[st][swz_off(r, cp + 1)]);
            bfr[tn] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
#pragma unroll
        for (int tm = 0; tm < 4; ++tm) {
            const int r = wm * 64 + tm * 16 + (lane & 15);
            const uint4 lo = *reinterpret_cast<const uint4*>(&lds_a[st][swz_off(r, cp)]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&lds_a[st][swz_off(r, cp + 1)]);
            const v8i af = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            v4f p[4];
#pragma unroll
            for (int tn = 0; tn < 4; ++tn) p[tn] = mfma_group(af, bfr[tn]);
#pragma unroll
            for (int tn = 0; tn < 4; ++tn)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float s = ROW_SCALED_B ? s4[tm][v] * sbc[tn] : s4[tm][v];
                    acc[tm][tn][v] = fmaf(p[tn][v], s, acc[tm][tn][v]);
                }
        }
    }

    // epilogue: bf16, round to nearest even
#pragma unroll
    for (int tm = 0; tm < 4; ++tm)
#pragma unroll
        for (int v = 0; v < 4; ++v) {
            const int64_t r = i0 + wm * 64 + tm * 16 + qrow + v;
            if (r < I) {
#pragma unroll
                for (int tn = 0; tn < 4; ++tn)
                    Cout[r * J + j0 + wn * 64 + tn * 16 + qcol] = (uint16_t)f32_to_bf16_rne(acc[tm][tn][v]);
            }
        }
}

template <bool ROW_SCALED_B>
static hipError_t launch_large(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, uint16_t* C,
                               int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg, hipStream_t st) {
    const int tiles_m = (int)((I + L_BM - 1) / L_BM), tiles_n = (int)(J / L_BN);
    hipLaunchKernelGGL(gemm_large_kernel<ROW_SCALED_B>, dim3(tiles_m * tiles_n), dim3(L_THREADS), 0, st, A, As, B,
                       Bs, C, I, J, Kc, sbj, sbg, tiles_m, tiles_n);
    return hipGetLastError();
}

hipError_t launch_gemm_block_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                      uint16_t* C, int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg,
                                      hipStream_t st) {
    return launch_large<false>(A, As, B, Bs, C, I, J, Kc, sbj, sbg, st);
}

hipError_t launch_gemm_row_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                    uint16_t* C, int64_t I, int64_t J, int64_t Kc, hipStream_t st) {
    return launch_large<true>(A, As, B, Bs, C, I, J, Kc, 0, 0, st);
}

}  // namespace jetfp8
