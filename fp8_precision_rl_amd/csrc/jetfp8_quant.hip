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

// 16 lanes own one 1x128 group (8 bf16 per lane, one 16-byte load); a 256-thread block owns the same
// group column of 16 consecutive rows, so the 16 scales it writes are contiguous.
__global__ __launch_bounds__(256) void quant_rows_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                         uint8_t* __restrict__ q, float* __restrict__ s) {
    const int lane16 = threadIdx.x & 15;
    const int64_t row = (int64_t)blockIdx.x * 16 + (threadIdx.x >> 4);
    const int64_t g = blockIdx.y;
    const bool live = row < R;
    uint4 v = make_uint4(0, 0, 0, 0);
    const int64_t off = row * C + g * 128 + lane16 * 8;
    if (live) v = *reinterpret_cast<const uint4*>(x + off);
    float f[8];
    f[0] = bf16_to_f32(v.x & 0xFFFFu); f[1] = bf16_to_f32(v.x >> 16);
    f[2] = bf16_to_f32(v.y & 0xFFFFu); f[3] = bf16_to_f32(v.y >> 16);
    f[4] = bf16_to_f32(v.z & 0xFFFFu); f[5] = bf16_to_f32(v.z >> 16);
    f[6] = bf16_to_f32(v.w & 0xFFFFu); f[7] = bf16_to_f32(v.w >> 16);
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) a = fmaxf(a, fabsf(f[i]));
#pragma unroll
    for (int m = 8; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 16));
    const GroupScale gs = make_group_scale(a);
    uint2 out;
    out.x = encode4(f[0], f[1], f[2], f[3], gs);
    out.y = encode4(f[4], f[5], f[6], f[7], gs);
    if (live) {
        *reinterpret_cast<uint2*>(q + off) = out;
        if (lane16 == 0) s[g * R + row] = gs.s;
    }
}

// One block owns a 128-row x 64-column tile: it stages the tile in LDS, reduces each column's 128
// values, and writes the codes transposed (each column becomes 128 contiguous bytes of the output).
__global__ __launch_bounds__(256) void quant_cols_t_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           uint8_t* __restrict__ qT, float* __restrict__ sT) {
    __shared__ uint16_t tile[128][64 + 2];
    __shared__ float red[4][64];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * 128;
    const int64_t c0 = (int64_t)blockIdx.x * 64;
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int id = t + 256 * i;           // 1024 chunks of 8 bf16: 128 rows x 8 chunks
        const int row = id >> 3, ch = id & 7;
        const uint4 v = *reinterpret_cast<const uint4*>(x + (r0 + row) * C + c0 + ch * 8);
        uint32_t* dst = reinterpret_cast<uint32_t*>(&tile[row][ch * 8]);
        dst[0] = v.x; dst[1] = v.y; dst[2] = v.z; dst[3] = v.w;
    }
    __syncthreads();
    const int col = t & 63, part = t >> 6;    // 4 parts of 32 rows each
    float f[32];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 32; ++i) {
        f[i] = bf16_to_f32(tile[part * 32 + i][col]);
        a = fmaxf(a, fabsf(f[i]));
    }
    red[part][col] = a;
    __syncthreads();
    a = fmaxf(fmaxf(red[0][col], red[1][col]), fmaxf(red[2][col], red[3][col]));
    const GroupScale gs = make_group_scale(a);
    uint32_t w[8];
#pragma unroll
    for (int i = 0; i < 8; ++i) w[i] = encode4(f[4 * i], f[4 * i + 1], f[4 * i + 2], f[4 * i + 3], gs);
    uint8_t* dst = qT + (c0 + col) * R + r0 + part * 32;
    reinterpret_cast<uint4*>(dst)[0] = make_uint4(w[0], w[1], w[2], w[3]);
    reinterpret_cast<uint4*>(dst)[1] = make_uint4(w[4], w[5], w[6], w[7]);
    if (part == 0) sT[(int64_t)blockIdx.y * C + c0 + col] = gs.s;
}

// One block owns one 128x128 block: 8 rows x 8 columns per thread, a block-wide amax, codes written in
// place and, through an LDS transpose, to the transposed copy.
__global__ __launch_bounds__(256) void quant_blocks_kernel(const uint16_t* __restrict__ x, int64_t R, int64_t C,
                                                           uint8_t* __restrict__ q, float* __restrict__ s,
                                                           uint8_t* __restrict__ qT) {
    __shared__ float wred[4];
    __shared__ uint8_t codes[128][128 + 4];
    const int t = threadIdx.x;
    const int64_t r0 = (int64_t)blockIdx.y * 128, c0 = (int64_t)blockIdx.x * 128;
    const int ch = t & 15;                    // 16-byte chunk within a 256-byte row
    float f[8][8];
    float a = 0.0f;
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (t >> 4) + 16 * i;
        const uint4 v = *reinterpret_cast<const uint4*>(x + (r0 + row) * C + c0 + ch * 8);
        f[i][0] = bf16_to_f32(v.x & 0xFFFFu); f[i][1] = bf16_to_f32(v.x >> 16);
        f[i][2] = bf16_to_f32(v.y & 0xFFFFu); f[i][3] = bf16_to_f32(v.y >> 16);
        f[i][4] = bf16_to_f32(v.z & 0xFFFFu); f[i][5] = bf16_to_f32(v.z >> 16);
        f[i][6] = bf16_to_f32(v.w & 0xFFFFu); f[i][7] = bf16_to_f32(v.w >> 16);
#pragma unroll
        for (int j = 0; j < 8; ++j) a = fmaxf(a, fabsf(f[i][j]));
    }
#pragma unroll
    for (int m = 32; m >= 1; m >>= 1) a = fmaxf(a, __shfl_xor(a, m, 64));
    if ((t & 63) == 0) wred[t >> 6] = a;
    __syncthreads();
    a = fmaxf(fmaxf(wred[0], wred[1]), fmaxf(wred[2], wred[3]));
    const GroupScale gs = make_group_scale(a);
#pragma unroll
    for (int i = 0; i < 8; ++i) {
        const int row = (t >> 4) + 16 * i;
        uint2 out;
        out.x = encode4(f[i][0], f[i][1], f[i][2], f[i][3], gs);
        out.y = encode4(f[i][4], f[i][5], f[i][6], f[i][7], gs);
        *reinterpret_cast<uint2*>(q + (r0 + row) * C + c0 + ch * 8) = out;
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

hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, hipStream_t st) {
    dim3 grid((unsigned)((R + 15) / 16), (unsigned)(C / 128));
    hipLaunchKernelGGL(quant_rows_kernel, grid, dim3(256), 0, st, x, R, C, q, s);
    return hipGetLastError();
}

hipError_t launch_quant_cols_t(const uint16_t* x, int64_t R, int64_t C, uint8_t* qT, float* sT, hipStream_t st) {
    // C is a multiple of 128, so of 64; R a multiple of 128.
    dim3 grid((unsigned)(C / 64), (unsigned)(R / 128));
    hipLaunchKernelGGL(quant_cols_t_kernel, grid, dim3(256), 0, st, x, R, C, qT, sT);
    return hipGetLastError();
}

hipError_t launch_quant_blocks(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT,
                               hipStream_t st) {
    dim3 grid((unsigned)(C / 128), (unsigned)(R / 128));
    hipLaunchKernelGGL(quant_blocks_kernel, grid, dim3(256), 0, st, x, R, C, q, s, qT);
    return hipGetLastError();
}

}  // namespace jetfp8
