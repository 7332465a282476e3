// Group quantization kernels (bf16 -> OCP E4M3 codes + fp32 scales) for gfx950.
//
// Groupings of the Jet-RL unified FP8 flow (Jet-RL explainers, "Schema de Quantification"):
//   rows   : 1x128 groups along the contiguous axis (activations, dY for DGrad)
//   cols_t : 128x1 groups along the row axis, codes written transposed (dY and X for WGrad)
//   blocks : 128x128 blocks (weights), optional transposed code copy for DGrad
// All three are HBM-streaming kernels: 2 bytes read and 1 byte (+1 for the transposed copy) written per
// element, plus 4 bytes per group of scale.
#include "jetfp8_common.h"
#include "jetfp8_launch.h"

namespace jetfp8 {

typedef __amdgpu_buffer_rsrc_t rsrc_q_t;
typedef unsigned int u32x4_q __attribute__((ext_vector_type(4)));
typedef unsigned int u32x2_q __attribute__((ext_vector_type(2)));

// 16-byte load (plain: measured faster than non-temporal loads for these access patterns on gfx950).
__device__ __forceinline__ uint4 load16(const uint16_t* p) { return *reinterpret_cast<const uint4*>(p); }

__device__ __forceinline__ void unpack8(const uint4& v, float f[8]) {
    f[0] = bf16_to_f32(v.x & 0xFFFFu); f[1] = bf16_to_f32(v.x >> 16);
    f[2] = bf16_to_f32(v.y & 0xFFFFu); f[3] = bf16_to_f32(v.y >> 16);
    f[4] = bf16_to_f32(v.z & 0xFFFFu); f[5] = bf16_to_f32(v.z >> 16);
    f[6] = bf16_to_f32(v.w & 0xFFFFu); f[7] = bf16_to_f32(v.w >> 16);
}

// 1x128 groups.  A block of QR_WAVES waves owns a tile of 32 rows x 512 columns (4 groups per row; for calls of
// at most 64 rows 8 rows, one per wave, which spreads a decode batch over 4 times as many blocks: measured 5.2 ->
// 4.3 us at 32 x 4096, the same codes): each
// wave reads 1 KB runs of one row (16 lanes per group, 8 bf16 per lane) and writes 512-byte runs of codes;
// the tile's 4 x 32 scales are written as four whole 128-byte lines.  All loads of a thread are issued
// before the first is used, unconditionally: lanes past the last row or column load an in-bounds stand-in
// (row R-1, column 0) and store nothing, so no branch separates the loads.  Blocks are numbered along the
// columns first.
constexpr int QR_ROWS = 32, QR_COLS = 512, QR_WAVES = 8;
#ifndef QR_SMALL_ROWS
#define QR_SMALL_ROWS 64
#endif

template <int QR_PASSES>
__global__ __launch_bounds__(QR_WAVES * 64) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t R,
                                                                   int64_t C, uint8_t* __restrict__ q,
                                                                   float* __restrict__ s, uint32_t col_blocks) {
    constexpr int QR_ROWS = QR_WAVES * QR_PASSES;
    __shared__ float sc[4][QR_ROWS];
    const int t = threadIdx.x, wave = __builtin_amdgcn_readfirstlane(t >> 6), lane = t & 63;
    const int gl = lane >> 4, lane16 = lane & 15;
    const uint32_t cb = blockIdx.x % col_blocks, rb = blockIdx.x / col_blocks;
    const int64_t c0 = (int64_t)cb * QR_COLS, r0 = (int64_t)rb * QR_ROWS;
    const int64_t col = c0 + gl * 128 + lane16 * 8;
    const bool col_ok = col < C;       // C is a multiple of 128: a group is wholly inside or outside
    const int64_t lcol = col_ok ? col : 0;
    uint4 v[QR_PASSES];
#pragma unroll
    for (int p = 0; p < QR_PASSES; ++p) {
        const int64_t row = min(r0 + p * QR_WAVES + wave, R - 1);
        v[p] = load16(x + row * C + lcol);
    }
#pragma unroll
    for (int p = 0; p < QR_PASSES; ++p) {
        const int64_t row = r0 + p * QR_WAVES + wave;
        float f[8];
        unpack8(v[p], f);
        const GroupScale gs = make_group_scale(bf16_to_f32(row16_max_u32(amax8_bits(v[p]))));
        const uint2 out = encode8(f, gs);
        if (col_ok && row < R) *reinterpret_cast<uint2*>(q + row * C + col) = out;
        if (lane16 == 0) sc[gl][p * QR_WAVES + wave] = gs.s;
    }
    __syncthreads();
    if (t < 4 * QR_ROWS) {
        const int g = t / QR_ROWS, r = t % QR_ROWS;
        const int64_t gg = c0 / 128 + g;
        if (gg * 128 < C && r0 + r < R) s[gg * R + r0 + r] = sc[g][r];
    }
}

// 128x1 groups, codes transposed.  A 256-thread block owns a 128-row x 128-column tile.
// Lane l of DPP row k (16 lanes) of wave w loads the 8x8 sub-tile of rows 8l .. 8l+7 and columns
// 32w + 8k .. +7 (eight 16-byte loads, all issued first), so each column's 128-row group is spread over
// the 16 lanes of one DPP row: a column's amax is a 16-lane row reduction, and the lane then holds 8
// consecutive rows of each of its 8 columns -- 8 bytes of the transposed output each, and the row's 16
// lanes write 128 contiguous bytes of a transposed row.  Lane j of a DPP row forms column j's scale and
// shares it through the wave's own LDS slots (every lane used to form all 8: 319.9 -> 312.0 us at
// 65536 x 7168, the same bits).
__global__ __launch_bounds__(256) void quant_cols_t_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           uint8_t* __restrict__ qT, float* __restrict__ sT,
                                                           uint32_t col_blocks) {
    // (s, r, p2, rcp) of the 8 columns of each DPP row, formed by lane j of the row for its column j
    __shared__ float4 cscale[4][4][8];
    const int t = threadIdx.x, lane = t & 63, wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l = lane & 15, k = lane >> 4;
    const uint32_t cb = blockIdx.x % col_blocks, rb = blockIdx.x / col_blocks;
    const int64_t r0 = (int64_t)rb * 128;
    const int64_t c = (int64_t)cb * 128 + wave * 32 + k * 8;     // first of this lane's 8 columns
    const bool ok = c < C;                                         // C is a multiple of 64, so of 8
    const int64_t lc = ok ? c : 0;                                 // in-bounds stand-in: loaded, never stored
    const uint16_t* xp = x + (r0 + 8 * l) * C + lc;                // the lane's first row; rows i at + i C
    uint4 v[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) v[i] = load16(xp + i * C);
    // column j of the sub-tile: element i is the 16-bit half (j & 1) of word (j >> 1) of v[i]
    auto elem = [&](int i, int j) -> float {
        const uint32_t w = (j >> 1) == 0 ? v[i].x : (j >> 1) == 1 ? v[i].y : (j >> 1) == 2 ? v[i].z : v[i].w;
        return bf16_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
    };
    // per-lane magnitude maxima of the 8 columns, two columns per word
    uint32_t cm[4];
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        auto word = [&](int i) { return w == 0 ? v[i].x : w == 1 ? v[i].y : w == 2 ? v[i].z : v[i].w; };
        cm[w] = pkmax16(pkmax16(max_mag2(word(0), word(1)), max_mag2(word(2), word(3))),
                        pkmax16(max_mag2(word(4), word(5)), max_mag2(word(6), word(7))));
    }
    // column amaxima over the DPP row (every lane ends with all 8), then lane j forms column j's scale
    uint32_t am[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) am[j] = row16_max_u32((j & 1) ? (cm[j >> 1] >> 16) : (cm[j >> 1] & 0xFFFFu));
    {
        const uint32_t mine = l == 0 ? am[0] : l == 1 ? am[1] : l == 2 ? am[2] : l == 3 ? am[3] :
                              l == 4 ? am[4] : l == 5 ? am[5] : l == 6 ? am[6] : am[7];
        if (l < 8) {
            const GroupScale gs = make_group_scale(bf16_to_f32(mine));
            cscale[wave][k][l] = make_float4(gs.s, gs.r, gs.p2, gs.rcp);
            // lanes 0..7 of each DPP row hold the scales of its 8 columns: 32 contiguous bytes per row
            if (ok) sT[(int64_t)rb * C + c + l] = gs.s;
        }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
    uint8_t* qp = qT + c * R + r0 + 8 * l;
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float f[8];
#pragma unroll
        for (int i = 0; i < 8; ++i) f[i] = elem(i, j);
        const float4 cs = cscale[wave][k][j];
        GroupScale gs;
        gs.s = cs.x;
        gs.r = cs.y;
        gs.p2 = cs.z;
        gs.rcp = cs.w;
        gs.tiny = cs.z != 1.0f;
        const uint2 out = encode8(f, gs);
        if (ok) *reinterpret_cast<uint2*>(qp + j * R) = out;
    }
}

// Four codes of one group packed little-endian into a uint32: encode8's arithmetic (fast quotient, per-element
// midpoint screen, exact fix of a screened element) on four elements.
__device__ __forceinline__ uint32_t encode4(const float x[4], const GroupScale& g) {
    constexpr uint32_t kSmall = 2u * (0x3C800000u + 3u) - 2u;    // (2 |q| pattern - 2) <= kSmall: 0 < |q| <= 2^-6 + 3 ulps
    float q[4];
    uint32_t smin = 0xFFFFFFFFu;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        q[i] = x[i] * g.rcp;
        smin = min(smin, (__float_as_uint(q[i]) << 1) - 2u);    // +-0 wraps to the top
    }
    if (g.tiny) {
#pragma unroll
        for (int i = 0; i < 4; ++i) q[i] = approx_quotient(x[i], g);
        smin = 0;
    }
    uint32_t k_mid;
    asm("s_mov_b32 %0, 0xfff80004" : "=s"(k_mid));
    if (smin <= kSmall) {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const uint32_t b = __float_as_uint(q[i]);
            const bool small = (b << 1) - 2u <= kSmall;
            if (small || ((b + k_mid) << 12) <= (8u << 12)) q[i] = resolve_at_midpoint(x[i], cell_midpoint(q[i], small), g);
        }
    } else {
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            if (((__float_as_uint(q[i]) + k_mid) << 12) <= (8u << 12))
                q[i] = resolve_at_midpoint(x[i], cell_midpoint(q[i], false), g);
        }
    }
    return cvt2_e4m3<true>(q[2], q[3], cvt2_e4m3<false>(q[0], q[1], __float_as_uint(q[1])));
}

// 1x128 and 128x1 groups of the same tensor from one read (the activation / gradient feeding a forward or DGrad
// GEMM and a WGrad GEMM): codes q [R][C] with scales s [C/128][R], and transposed codes qT [C][R] with scales
// sT [R/128][C].  A 512-thread block owns a 128x128 tile, so each of its rows is one 1x128 group and each of its
// columns one 128x1 group.  Lane l of DPP row k of wave w holds the 4x8 sub-tile of rows 16 w + 4 k .. +3 and
// columns 8 l .. +7 (four 16-byte loads; a DPP row reads 256 contiguous bytes of each of its rows):
//   - a row's group lies in one DPP row: its amax is a 16-lane row reduction, and the 16 lanes write the row's
//     128 codes as one contiguous run;
//   - a column's group spans the whole block: per-lane maxima, then across the wave's four DPP rows, then
//     across the eight waves through LDS; each lane encodes its four values of each of its 8 columns into one
//     word, the words are staged in LDS and leave as whole 128-byte transposed rows;
//   - each group's scale (and its reciprocal) is formed once, by one lane, and read from LDS by the lanes that
//     encode with it (a row's 16 lanes, a column's 32).
// 4x8 sub-tiles instead of 8x8 ones in 256-thread blocks (96 VGPRs capped, 5 waves per SIMD) hold half the values
// per lane, and forming each scale once drops the per-lane scale arithmetic: 49 VGPRs, 8 waves per SIMD.
// Bitwise the same codes; measured on 65536-row tensors 4.20 -> 4.87 TB/s at x 5120, 4.64 -> 4.94 at dY 7168,
// and 4.39 -> 4.70 at x 27648.
// Memory access goes through raw buffer descriptors built from block-uniform bases (scalar registers) with
// 32-bit lane offsets, so no 64-bit address arithmetic runs on the vector unit.  A descriptor spans exactly
// the bytes its accesses touch; the launcher checks that every span and offset fits in 31 bits.
__device__ __forceinline__ rsrc_q_t span_rsrc(const void* base, int64_t bytes) {
    return __builtin_amdgcn_make_buffer_rsrc(const_cast<void*>(base), (short)0, (int)bytes, 0x00020000);
}

// Word index in row c of the transposed-code staging buffer for logical word w (0..31): its 16-byte chunk w / 4 is
// XORed with the row's 8-column group (c / 8) % 8, so a staging write instruction (16 columns 8 apart) covers all
// eight chunks.
__device__ __forceinline__ int tcode_word(int c, int w) { return (((w >> 2) ^ ((c >> 3) & 7)) << 2) | (w & 3); }

__global__ __launch_bounds__(512) __attribute__((amdgpu_waves_per_eu(6, 8))) void quant_dual_kernel(
    const uint16_t* __restrict__ x, int64_t R, int64_t C, uint8_t* __restrict__ q, float* __restrict__ s,
    uint8_t* __restrict__ qT, float* __restrict__ sT, uint32_t col_blocks) {
    __shared__ uint32_t red[8][16][4];
    __shared__ float4 cscale[8][16];         // (s, r, p2, rcp) of column 8 l + j at [j][l]: a read of one j by
                                             // the 16 lanes of a DPP row covers 256 contiguous bytes
    __shared__ float4 rscale[8][16];         // the same for each wave's 16 rows
    // [column][4-row word] with the 16-byte chunks of a row XOR-swizzled by the column's 8-column group
    // (tcode_word): rows stay 16-byte aligned, so the transposed rows come out as 16-byte reads, and the 16 lanes
    // of a write instruction spread over the banks.
    __shared__ __attribute__((aligned(16))) uint32_t tcodes[128][32];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l16 = lane & 15, rs = lane >> 4, rb4 = 4 * wave + rs;     // rb4: the lane's 4-row word of a column
    const uint32_t cb = blockIdx.x % col_blocks, rb = blockIdx.x / col_blocks;
    const int64_t r0 = (int64_t)rb * 128, c0 = (int64_t)cb * 128;
    // this wave's 16 rows start at wr; the lane's 4x8 sub-tile is rows wr + 4 rs .. +3, columns c0 + 8 l16 ..
    const int64_t wr = r0 + 16 * wave;
    const int Ci = (int)C;
    const int64_t span = 15 * C + 128;                       // elements from (wr, c0) to (wr + 15, c0 + 127)
    const rsrc_q_t rx = span_rsrc(x + wr * C + c0, 2 * span);
    const rsrc_q_t rq = span_rsrc(q + wr * C + c0, span);
    const int lo = 4 * rs * Ci + 8 * l16;                    // element offset of the lane's first row
    uint4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const u32x4_q w = __builtin_amdgcn_raw_buffer_load_b128(rx, 2 * lo, 2 * i * Ci, 0);
        v[i] = make_uint4(w[0], w[1], w[2], w[3]);
    }

    // magnitude maxima from the sign-cleared words: per row of the sub-tile (8 values) and per column (two
    // columns per word, over the 4 rows); the column maxima then over the wave's 4 DPP rows
    uint32_t cm[4] = {0u, 0u, 0u, 0u}, rmax[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const uint32_t m0 = mag2(v[i].x), m1 = mag2(v[i].y), m2 = mag2(v[i].z), m3 = mag2(v[i].w);
        cm[0] = pkmax16(cm[0], m0);
        cm[1] = pkmax16(cm[1], m1);
        cm[2] = pkmax16(cm[2], m2);
        cm[3] = pkmax16(cm[3], m3);
        const uint32_t r = pkmax16(pkmax16(m0, m1), pkmax16(m2, m3));
        rmax[i] = max(r & 0xFFFFu, r >> 16);
    }
#pragma unroll
    for (int w = 0; w < 4; ++w) {
        cm[w] = pkmax16(cm[w], (uint32_t)__shfl_xor((int)cm[w], 16, 64));
        cm[w] = pkmax16(cm[w], (uint32_t)__shfl_xor((int)cm[w], 32, 64));
    }
    if (rs == 0) {
#pragma unroll
        for (int w = 0; w < 4; ++w) red[wave][l16][w] = cm[w];
    }

    // 1x128 groups: one per row; lane i of each DPP row forms the scale of its row i (i < 4) for the 16 lanes
    {
        uint32_t am[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) am[i] = row16_max_u32(rmax[i]);
        const uint32_t mine = l16 == 0 ? am[0] : l16 == 1 ? am[1] : l16 == 2 ? am[2] : am[3];
        if (l16 < 4) {
            const GroupScale gs = make_group_scale(bf16_to_f32(mine));
            rscale[wave][4 * rs + l16] = make_float4(gs.s, gs.r, gs.p2, gs.rcp);
            s[(c0 / 128) * R + wr + (4 * rs + l16)] = gs.s;
        }
    }
    __builtin_amdgcn_wave_barrier();
    asm volatile("" ::: "memory");
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        float f[8];
        unpack8(v[i], f);
        const float4 cs = rscale[wave][4 * rs + i];
        GroupScale gs;
        gs.s = cs.x;
        gs.r = cs.y;
        gs.p2 = cs.z;
        gs.rcp = cs.w;
        gs.tiny = cs.z != 1.0f;
        const uint2 out = encode8(f, gs);
        const u32x2_q o = {out.x, out.y};
        __builtin_amdgcn_raw_buffer_store_b64(o, rq, lo, i * Ci, 0);
    }

    // 128x1 groups: one per column; each column's scale formed once, by thread c
    __syncthreads();
    if (t < 128) {
        const int l = t >> 3, w = (t & 7) >> 1;
        const uint32_t a = pkmax16(pkmax16(red[0][l][w], red[1][l][w]), pkmax16(red[2][l][w], red[3][l][w]));
        const uint32_t b = pkmax16(pkmax16(red[4][l][w], red[5][l][w]), pkmax16(red[6][l][w], red[7][l][w]));
        const uint32_t m = pkmax16(a, b);
        const GroupScale gs = make_group_scale(bf16_to_f32((t & 1) ? (m >> 16) : (m & 0xFFFFu)));
        cscale[t & 7][t >> 3] = make_float4(gs.s, gs.r, gs.p2, gs.rcp);
        sT[(int64_t)rb * C + c0 + t] = gs.s;
    }
    __syncthreads();
    auto elem = [&](int i, int j) -> float {
        const uint32_t w = (j >> 1) == 0 ? v[i].x : (j >> 1) == 1 ? v[i].y : (j >> 1) == 2 ? v[i].z : v[i].w;
        return bf16_to_f32((j & 1) ? (w >> 16) : (w & 0xFFFFu));
    };
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = elem(i, j);
        const float4 cs = cscale[j][l16];
        GroupScale gs;
        gs.s = cs.x;
        gs.r = cs.y;
        gs.p2 = cs.z;
        gs.rcp = cs.w;
        gs.tiny = cs.z != 1.0f;
        tcodes[8 * l16 + j][tcode_word(8 * l16 + j, rb4)] = encode4(f, gs);
    }
    __syncthreads();
    // thread t writes bytes 32 (t & 3) .. +31 of transposed row c0 + t / 4 (rows r0 .. r0 + 127 of it)
    const rsrc_q_t rqt = span_rsrc(qT + c0 * R + r0, 127 * R + 128);
    const int oc = t >> 2, qt = t & 3;
    const int to = oc * (int)R + 32 * qt;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(&tcodes[oc][tcode_word(oc, 8 * qt + 4 * k)]);
        const u32x4_q o = {w4.x, w4.y, w4.z, w4.w};
        __builtin_amdgcn_raw_buffer_store_b128(o, rqt, to + 16 * k, 0, 0);
    }
}

// 128x1 groups of a saved FP8 activation (the pages keep the activations saved for the backward pass in FP8;
// WGrad groups X along the token axis): the 1x128 codes q [R][C] with their scales s [C/128][R] are
// dequantized, x' = fl32(decode(code) * s) with one fp32 product, and x' is quantized in 128x1 groups along R
// as the bf16 path does (the encode arithmetic and its exactness argument hold for any finite fp32 x').
// Output: qT [C][R], sT [R/128][C].  The work is laid out as in quant_dual_kernel: a 128x128 tile per 512-thread
// block, a 4x8 sub-tile per lane (4 rows x 8 codes), column maxima across the wave's DPP rows and the block's
// waves, each column scale formed once and shared through LDS, transposed codes staged in LDS.  (With 8x8
// sub-tiles in 256-thread blocks, 85 VGPRs and 5 waves per SIMD: 198.6 -> 167.0 us at 65536 x 5120 and 1200 ->
// 850 us at 65536 x 27648, bitwise the same.)  2 bytes of traffic per element instead of 3.
__global__ __launch_bounds__(512) void quant_requant_cols_kernel(const uint8_t* __restrict__ q,
                                                                 const float* __restrict__ s, int64_t R,
                                                                 int64_t C, uint8_t* __restrict__ qT,
                                                                 float* __restrict__ sT, uint32_t col_blocks) {
    __shared__ uint32_t red[8][16][8];
    __shared__ float4 cscale[8][16];         // (s, r, p2, rcp) of column 8 l + j at [j][l], as in quant_dual_kernel
    __shared__ __attribute__((aligned(16))) uint32_t tcodes[128][32];   // as in quant_dual_kernel
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int l16 = lane & 15, rs = lane >> 4, rb4 = 4 * wave + rs;
    const uint32_t cb = blockIdx.x % col_blocks, rb = blockIdx.x / col_blocks;
    const int64_t r0 = (int64_t)rb * 128, c0 = (int64_t)cb * 128;
    const int64_t wr = r0 + 16 * wave;
    const int Ci = (int)C;
    const rsrc_q_t rcodes = span_rsrc(q + wr * C + c0, 15 * C + 128);
    const int lo = 4 * rs * Ci + 8 * l16;
    u32x2_q cw[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) cw[i] = __builtin_amdgcn_raw_buffer_load_b64(rcodes, lo, i * Ci, 0);
    // saved scales of the lane's 4 rows (group c0 / 128 of each row): 16 contiguous bytes
    const float4 sa = *reinterpret_cast<const float4*>(s + (c0 / 128) * R + wr + 4 * rs);
    const float sr[4] = {sa.x, sa.y, sa.z, sa.w};

    // dequantize: element (i, j) is byte j of the lane's row i
    float xv[4][8];
#pragma unroll
    for (int i = 0; i < 4; ++i)
#pragma unroll
        for (int w = 0; w < 2; ++w) {
            const auto lo2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i][w], false);   // bytes 0, 1 of the word
            const auto hi2 = __builtin_amdgcn_cvt_pk_f32_fp8((int)cw[i][w], true);    // bytes 2, 3
            xv[i][4 * w] = lo2[0] * sr[i];
            xv[i][4 * w + 1] = lo2[1] * sr[i];
            xv[i][4 * w + 2] = hi2[0] * sr[i];
            xv[i][4 * w + 3] = hi2[1] * sr[i];
        }

    // column maxima of the magnitude bits (fp32 patterns order like the magnitudes): this lane's 4 rows, then
    // the wave's 4 DPP rows, then the block's 8 waves; each column's scale formed once, by thread c
    uint32_t cm[8];
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        uint32_t m = 0;
#pragma unroll
        for (int i = 0; i < 4; ++i) m = max(m, __float_as_uint(xv[i][j]) & 0x7FFFFFFFu);
        m = max(m, (uint32_t)__shfl_xor((int)m, 16, 64));
        m = max(m, (uint32_t)__shfl_xor((int)m, 32, 64));
        cm[j] = m;
    }
    if (rs == 0) {
#pragma unroll
        for (int j = 0; j < 8; ++j) red[wave][l16][j] = cm[j];
    }
    __syncthreads();
    if (t < 128) {
        const int l = t >> 3, j = t & 7;
        const uint32_t a = max(max(red[0][l][j], red[1][l][j]), max(red[2][l][j], red[3][l][j]));
        const uint32_t b = max(max(red[4][l][j], red[5][l][j]), max(red[6][l][j], red[7][l][j]));
        const GroupScale gs = make_group_scale(__uint_as_float(max(a, b)));
        cscale[j][l] = make_float4(gs.s, gs.r, gs.p2, gs.rcp);
        sT[(int64_t)rb * C + c0 + t] = gs.s;
    }
    __syncthreads();
#pragma unroll
    for (int j = 0; j < 8; ++j) {
        float f[4];
#pragma unroll
        for (int i = 0; i < 4; ++i) f[i] = xv[i][j];
        const float4 cs = cscale[j][l16];
        GroupScale gs;
        gs.s = cs.x;
        gs.r = cs.y;
        gs.p2 = cs.z;
        gs.rcp = cs.w;
        gs.tiny = cs.z != 1.0f;
        tcodes[8 * l16 + j][tcode_word(8 * l16 + j, rb4)] = encode4(f, gs);
    }
    __syncthreads();
    // thread t writes bytes 32 (t & 3) .. +31 of transposed row c0 + t / 4 (rows r0 .. r0 + 127 of it)
    const rsrc_q_t rqt = span_rsrc(qT + c0 * R + r0, 127 * R + 128);
    const int oc = t >> 2, qt = t & 3;
    const int to = oc * (int)R + 32 * qt;
#pragma unroll
    for (int k = 0; k < 2; ++k) {
        const uint4 w4 = *reinterpret_cast<const uint4*>(&tcodes[oc][tcode_word(oc, 8 * qt + 4 * k)]);
        const u32x4_q o = {w4.x, w4.y, w4.z, w4.w};
        __builtin_amdgcn_raw_buffer_store_b128(o, rqt, to + 16 * k, 0, 0);
    }
}

// One block owns one 128x128 block: 8 rows x 8 columns per thread, a block-wide amax, codes written in
// place and, through an LDS transpose, to the transposed copy.
// FRAG: the codes go out in the fragment order the small-M GEMM kernel loads (JETFP8_BLOCKS_128x128_FRAG): for each
// 16-row slice s and 128-column group g a 2 KB block at (s * C/128 + g) * 2048, in which lane l of a wave (row l % 16 of
// the slice, columns 32 (l / 16) .. +31 of the group) has columns +0..15 at 16 l and +16..31 at 1024 + 16 l.
template <bool FRAG>
__global__ __launch_bounds__(256) void quant_blocks_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           uint8_t* __restrict__ q, float* __restrict__ s,
                                                           uint8_t* __restrict__ qT) {
    __shared__ uint32_t wred[4];
    __shared__ uint8_t codes[128][128 + 4];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * 128, c0 = (int64_t)blockIdx.x * 128;
    const int ch = t & 15;                    // 16-byte chunk within a 256-byte row
    float f[8][8];
    uint32_t a = 0;      // magnitude maximum as a bf16 bit pattern (see amax8_bits)
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (t >> 4) + 16 * i;
        const uint4 v = load16(x + (r0 + row) * C + c0 + ch * 8);
        unpack8(v, f[i]);
        a = max(a, amax8_bits(v));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) a = max(a, (uint32_t)__shfl_xor((int)a, m, 64));
    if ((t & 63) == 0) wred[t >> 6] = a;
    __syncthreads();
    a = max(max(wred[0], wred[1]), max(wred[2], wred[3]));
    const GroupScale gs = make_group_scale(bf16_to_f32(a));
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (t >> 4) + 16 * i;
        const uint2 out = encode8(f[i], gs);
        if (FRAG) {
            // columns 8 ch .. +7 of the group: lane (row % 16) + 16 (ch / 4), half (ch % 4) / 2, byte 8 (ch % 2)
            const int64_t blk = ((r0 + row) / 16) * (C / 128) + c0 / 128;
            const int off = ((ch & 3) >> 1) * 1024 + 16 * ((row & 15) + 16 * (ch >> 2)) + 8 * (ch & 1);
            *reinterpret_cast<uint2*>(q + blk * 2048 + off) = out;
        } else {
            *reinterpret_cast<uint2*>(q + (r0 + row) * C + c0 + ch * 8) = out;
        }
        if (qT) {
            uint32_t* crow = reinterpret_cast<uint32_t*>(&codes[row][ch * 8]);
            crow[0] = out.x; crow[1] = out.y;
        }
    }
    if (t == 0) s[blockIdx.y * (C / 128) + blockIdx.x] = gs.s;
    if (qT) {
        __syncthreads();
        // transposed copy: thread t writes 64 bytes of output row (c0 + t/2), rows r0 + (t&1)*64 ...
        const int oc = t >> 1, half = t & 1;
        uint32_t w[16];
#pragma unroll
        for (int i = 0; i < 16; ++i) {
            const int rb = half * 64 + 4 * i;
            w[i] = (uint32_t)codes[rb][oc] | ((uint32_t)codes[rb + 1][oc] << 8) |
                   ((uint32_t)codes[rb + 2][oc] << 16) | ((uint32_t)codes[rb + 3][oc] << 24);
        }
        uint4* dst = reinterpret_cast<uint4*>(qT + (c0 + oc) * R + r0 + half * 64);
#pragma unroll
        for (int i = 0; i < 4; ++i) dst[i] = make_uint4(w[4 * i], w[4 * i + 1], w[4 * i + 2], w[4 * i + 3]);
    }
}

// One-dimensional grids of at most 2^31 - 1 blocks; the fused and requantizing kernels also address a tile's
// 32 (or 128) rows through buffer offsets below 2^31 bytes; the block kernel's grid.y (row blocks) is at most 65535.
bool quant_rows_fits(int64_t R, int64_t C) {
    return ((C + QR_COLS - 1) / QR_COLS) * ((R + QR_ROWS - 1) / QR_ROWS) <= 0x7FFFFFFF;
}
bool quant_cols_t_fits(int64_t R, int64_t C) { return ((C + 127) / 128) * (R / 128) <= 0x7FFFFFFF; }
bool quant_dual_fits(int64_t R, int64_t C) {
    return (C / 128) * (R / 128) <= 0x7FFFFFFF && 64 * C + 256 < ((int64_t)1 << 31) && 128 * R + 128 < ((int64_t)1 << 31);
}
bool quant_requant_cols_fits(int64_t R, int64_t C) {
    return (C / 128) * (R / 128) <= 0x7FFFFFFF && 32 * C + 128 < ((int64_t)1 << 31) && 128 * R + 128 < ((int64_t)1 << 31);
}
bool quant_blocks_fits(int64_t R, int64_t C) { return R / 128 <= 65535 && C / 128 <= 0x7FFFFFFF; }

hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, hipStream_t st) {
    const int64_t col_blocks = (C + QR_COLS - 1) / QR_COLS;
    if (!quant_rows_fits(R, C)) return hipErrorInvalidConfiguration;
    if (R <= QR_SMALL_ROWS) {
        // decode-sized calls: one row per wave, so a 32-row call spreads over 4 times as many blocks
        const int64_t row_blocks = (R + QR_WAVES - 1) / QR_WAVES;
        hipLaunchKernelGGL(quant_rows_kernel<1>, dim3((unsigned)(col_blocks * row_blocks)), dim3(QR_WAVES * 64), 0, st,
                           x, R, C, q, s, (uint32_t)col_blocks);
    } else {
        const int64_t row_blocks = (R + QR_ROWS - 1) / QR_ROWS;
        hipLaunchKernelGGL(quant_rows_kernel<QR_ROWS / QR_WAVES>, dim3((unsigned)(col_blocks * row_blocks)),
                           dim3(QR_WAVES * 64), 0, st, x, R, C, q, s, (uint32_t)col_blocks);
    }
    return hipGetLastError();
}

hipError_t launch_quant_cols_t(const uint16_t* x, int64_t R, int64_t C, uint8_t* qT, float* sT, hipStream_t st) {
    // R is a multiple of 128 (whole groups); C a multiple of 64 (a partial last column tile is masked).
    const int64_t col_blocks = (C + 127) / 128, row_blocks = R / 128;
    if (!quant_cols_t_fits(R, C)) return hipErrorInvalidConfiguration;
    hipLaunchKernelGGL(quant_cols_t_kernel, dim3((unsigned)(col_blocks * row_blocks)), dim3(256), 0, st, x, R, C, qT,
                       sT, (uint32_t)col_blocks);
    return hipGetLastError();
}

hipError_t launch_quant_dual(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT, float* sT,
                             hipStream_t st) {
    // R and C are multiples of 128 (whole groups both ways)
    const int64_t col_blocks = C / 128, row_blocks = R / 128;
    // buffer spans and offsets in 31 bits: a wave's 16 bf16 rows (2 (15 C + 128) bytes; the check allows 32) and
    // 128 transposed rows
    if (!quant_dual_fits(R, C)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_dual_kernel, dim3((unsigned)(col_blocks * row_blocks)), dim3(512), 0, st, x, R, C, q, s,
                       qT, sT, (uint32_t)col_blocks);
    return hipGetLastError();
}

hipError_t launch_quant_requant_cols(const uint8_t* q, const float* s, int64_t R, int64_t C, uint8_t* qT,
                                     float* sT, hipStream_t st) {
    // R and C are multiples of 128; buffer spans and offsets in 31 bits (32 code rows, 128 transposed rows)
    const int64_t col_blocks = C / 128, row_blocks = R / 128;
    if (!quant_requant_cols_fits(R, C)) return hipErrorInvalidValue;
    hipLaunchKernelGGL(quant_requant_cols_kernel, dim3((unsigned)(col_blocks * row_blocks)), dim3(512), 0, st, q, s,
                       R, C, qT, sT, (uint32_t)col_blocks);
    return hipGetLastError();
}

hipError_t launch_quant_blocks(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT, bool frag,
                               hipStream_t st) {
    if (!quant_blocks_fits(R, C)) return hipErrorInvalidValue;
    dim3 grid((unsigned)(C / 128), (unsigned)(R / 128));
    if (frag) hipLaunchKernelGGL(quant_blocks_kernel<true>, grid, dim3(256), 0, st, x, R, C, q, s, qT);
    else hipLaunchKernelGGL(quant_blocks_kernel<false>, grid, dim3(256), 0, st, x, R, C, q, s, qT);
    return hipGetLastError();
}

}  // namespace jetfp8
