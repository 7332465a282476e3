// Host-side launchers of the libjetfp8 kernels (shapes are validated by the C ABI layer before these run).
#pragma once
#include <hip/hip_runtime.h>
#include <stdint.h>

namespace jetfp8 {

// The GEMM kernels address a block's operand band (256 rows x contraction bytes) and a scale array
// (groups x rows x 4 bytes) through 32-bit buffer offsets; the C ABI rejects shapes beyond this.
constexpr int64_t kMaxGemmBand = ((int64_t)1 << 31) - 1;

// Size limits of each kernel's launch grid and of its 32-bit buffer offsets.  The C ABI checks these on the host
// (JETFP8_ERR_SHAPE) before calling a launcher; the launchers assume them.
bool quant_rows_fits(int64_t R, int64_t C);
bool quant_cols_t_fits(int64_t R, int64_t C);
bool quant_dual_fits(int64_t R, int64_t C);
bool quant_requant_cols_fits(int64_t R, int64_t C);
bool quant_blocks_fits(int64_t R, int64_t C);
bool swiglu_quant_fits(int64_t R, int64_t F);

hipError_t launch_quant_rows(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, hipStream_t st);
hipError_t launch_quant_cols_t(const uint16_t* x, int64_t R, int64_t C, uint8_t* qT, float* sT, hipStream_t st);
hipError_t launch_quant_dual(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT, float* sT,
                             hipStream_t st);
hipError_t launch_quant_requant_cols(const uint8_t* q, const float* s, int64_t R, int64_t C, uint8_t* qT,
                                     float* sT, hipStream_t st);
// Fused producers (1x128 codes of the produced bf16 activation).  RMSNorm holds a row in registers: at most
// kRmsNormMaxCols columns.
constexpr int64_t kRmsNormMaxCols = 8192;
hipError_t launch_rmsnorm_quant(const uint16_t* x, const uint16_t* w, int64_t R, int64_t C, float eps, uint8_t* q,
                                float* s, float* rstd, uint16_t* y, hipStream_t st);
hipError_t launch_swiglu_quant(const uint16_t* gu, int64_t R, int64_t F, uint8_t* q, float* s, uint16_t* h,
                               hipStream_t st);
// frag = true: q in the fragment order of JETFP8_BLOCKS_128x128_FRAG instead of row-major.
hipError_t launch_quant_blocks(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, uint8_t* qT, bool frag,
                               hipStream_t st);

// C[i][j] = sum_g As[g][i] * sb(j, g) * sum_{k in g} A[i][k] * B[j][k], A [I][Kc], B [J][Kc].
// Block-scaled B: sb(j, g) = Bs[(j / 128) * sbj + g * sbg].  Row-scaled B: sb(j, g) = Bs[g * J + j].
hipError_t launch_gemm_block_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                      uint16_t* C, int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg,
                                      hipStream_t st);
// Rows r0 .. r0 + rows - 1 of a block-scaled-B GEMM with I rows on the small-M kernel (decode_rows_fit(rows, Kc)).
bool decode_rows_fit(int64_t rows, int64_t Kc);
hipError_t launch_decode_rows(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, uint16_t* C,
                              int64_t I, int64_t r0, int64_t rows, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg,
                              hipStream_t st);
// Forward GEMM with the weight codes in the fragment order of JETFP8_BLOCKS_128x128_FRAG (small-M kernel only:
// M <= 64 and (K / 128) * M <= 8192, checked by gemm_fwd_frag_fits).
bool gemm_fwd_frag_fits(int64_t M, int64_t K);
hipError_t launch_gemm_fwd_frag(const uint8_t* xq, const float* xs, const uint8_t* wqf, const float* ws, uint16_t* y,
                                int64_t M, int64_t N, int64_t K, hipStream_t st);
hipError_t launch_gemm_row_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                    uint16_t* C, int64_t I, int64_t J, int64_t Kc, hipStream_t st);

}  // namespace jetfp8
