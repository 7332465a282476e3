/*
 * jetfp8.h -- C ABI of the MI355X (gfx950) FP8 group-quantize + block-scaled GEMM library.
 *
 * The operations are those of the Jet-RL unified FP8 precision flow ("Jet-RL: Enabling On-Policy FP8
 * Reinforcement Learning with Unified Training and Rollout Precision Flow", gist.science explainers,
 * sections "Architecture Centrale" and "Schema de Quantification" / "Esquema de Quantizacao"):
 * the same FP8 linear layers serve rollout and the training forward; activations are quantized in 1x128
 * groups, weights in 128x128 blocks; gradients between operators stay BF16 and are quantized inside the
 * DGrad and WGrad GEMMs, which run in FP8 ("1x128 and 128x1" groupings for WGrad).
 *
 * Numerics (readings of what the pages leave open):
 *   FP8 format ... OCP E4M3 (bias 7, largest finite 448, NaN never produced).
 *   scale ........ s = fl32(amax / 448) per group, computed on every call (no calibration state).
 *   code ......... nearest E4M3 value to x / s (exact quotient), ties to the even code, |x/s| > 448
 *                  saturates to 448; an all-zero group has s = 0 and signed-zero codes.
 *   GEMMs ........ per output element: acc = +0; for each 128-wide group g of the contraction axis in
 *                  ascending order: acc = fma(p_g, fl32(sa_g * sb_g), acc), where p_g is the fp32 group
 *                  dot product formed by one gfx950 FP8 matrix instruction; out = bf16(acc), round to
 *                  nearest even.  The contraction is never split, so an output row is bitwise the same
 *                  whatever the number of rows in the call (decode M=1 and a training batch agree).
 *
 * Conventions for every entry point:
 *   - Matrices are dense, row-major, last index contiguous; bf16 tensors are passed as raw 16-bit
 *     patterns (void*), FP8 codes as uint8_t, scales as float.  No strides.
 *   - Every pointer is a DEVICE pointer owned by the caller; the library never allocates, frees or
 *     synchronizes.  Work is enqueued on `stream` (a hipStream_t; NULL = the default stream) and runs
 *     asynchronously; outputs are valid once the stream has reached that point.
 *   - Arguments are validated on the host before anything is launched.  Return value: JETFP8_OK, or a
 *     negative jetfp8_status; on error nothing has been enqueued and outputs are untouched
 *     (JETFP8_ERR_HIP: a launch was rejected by the runtime; earlier kernels of the same call may have
 *     been enqueued).  No exception ever crosses this interface.
 *   - All pointers must be 16-byte aligned (JETFP8_ERR_ALIGN otherwise).  Buffers must not overlap.
 *   - Sizes: every dimension >= 1; every grouped or contraction axis a multiple of 128, plus the
 *     per-mode rules below (JETFP8_ERR_SHAPE otherwise); every dimension < 2^31.  Kernels address their
 *     tiles with 32-bit offsets and launch one-dimensional grids, so each call also rejects, with
 *     JETFP8_ERR_SHAPE and before any launch:
 *       GEMMs ............... 256 * (contraction length) >= 2^31, or (contraction length / 128) * (rows of
 *                             either operand) * 4 >= 2^31 (bytes of a scale array);
 *       ROWS_1x128 .......... ceil(cols / 512) * ceil(rows / 32) > 2^31 - 1;
 *       COLS_128x1_T ........ ceil(cols / 128) * (rows / 128) > 2^31 - 1;
 *       BLOCKS_128x128 ...... rows / 128 > 65535;
 *       quantize_dual ....... (cols / 128) * (rows / 128) > 2^31 - 1, 64 * cols + 256 >= 2^31, or
 *                             128 * rows + 128 >= 2^31;
 *       requantize_cols_t ... (cols / 128) * (rows / 128) > 2^31 - 1, 32 * cols + 128 >= 2^31, or
 *                             128 * rows + 128 >= 2^31;
 *       swiglu_quantize ..... ceil(cols / 512) * ceil(rows / 32) >= 2^31, or 128 * cols >= 2^31 (32 rows of
 *                             gate_up in bytes).
 *   - Thread safety: calls are independent; concurrent calls on different streams are allowed.
 */
#ifndef JETFP8_H
#define JETFP8_H

#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    JETFP8_OK = 0,
    JETFP8_ERR_NULL = -1,   /* a required pointer is NULL */
    JETFP8_ERR_SHAPE = -2,  /* a dimension < 1, >= 2^31, or a grouped/contraction axis not a multiple of 128 */
    JETFP8_ERR_ALIGN = -3,  /* a pointer is not 16-byte aligned */
    JETFP8_ERR_MODE = -4,   /* unknown grouping mode, or dst_codes_t given for a mode without it */
    JETFP8_ERR_HIP = -5,    /* the HIP runtime rejected a launch */
    JETFP8_ERR_VALUE = -6   /* a scalar argument is outside its domain (e.g. eps <= 0) */
} jetfp8_status;

typedef enum {
    /* 1x128 groups along the contiguous axis (activations X for the forward, dY for DGrad).
     * src [rows][cols] -> dst_codes [rows][cols], dst_scales [cols/128][rows].  cols % 128 == 0. */
    JETFP8_ROWS_1x128 = 0,
    /* 128x1 groups along the row axis, codes written transposed (dY and X for WGrad, grouped along
     * the token axis).  src [rows][cols] -> dst_codes [cols][rows], dst_scales [rows/128][cols].
     * rows % 128 == 0, cols % 64 == 0. */
    JETFP8_COLS_128x1_T = 1,
    /* 128x128 blocks (weights).  src [rows][cols] -> dst_codes [rows][cols],
     * dst_scales [rows/128][cols/128], and when dst_codes_t != NULL the same codes transposed,
     * dst_codes_t [cols][rows] (the B operand of DGrad).  rows % 128 == 0 and cols % 128 == 0. */
    JETFP8_BLOCKS_128x128 = 2,
    /* As JETFP8_BLOCKS_128x128 (same codes, scales and optional row-major transposed copy), with dst_codes written
     * in the fragment order that jetfp8_gemm_fwd_frag reads: the byte of row n, column k goes to
     *   ((n / 16) * (cols / 128) + k / 128) * 2048 + ((k % 32) / 16) * 1024 + 16 * (n % 16 + 16 * ((k % 128) / 32))
     *   + k % 16.
     * A pure permutation of the row-major codes (same size); rows % 128 == 0 and cols % 128 == 0. */
    JETFP8_BLOCKS_128x128_FRAG = 3
} jetfp8_grouping;

/* Group quantization of a bf16 matrix to E4M3 codes plus fp32 scales (Jet-RL explainers,
 * "Schema de Quantification": 1x128 per-group for activations, 128x128 per-block for weights;
 * 1x128 and 128x1 for WGrad).  dst_codes_t is only accepted (and optional) for BLOCKS_128x128;
 * pass NULL for the other modes. */
int jetfp8_quantize(const void* src_bf16, int64_t rows, int64_t cols, int mode,
                    uint8_t* dst_codes, float* dst_scales, uint8_t* dst_codes_t, void* stream);

/* Both groupings of one bf16 matrix from a single read of it: the 1x128 codes and scales of
 * JETFP8_ROWS_1x128 and the transposed 128x1 codes and scales of JETFP8_COLS_128x1_T, bit for bit the
 * outputs of those two modes.  This serves a tensor that feeds a GEMM along its contiguous axis and the
 * WGrad GEMM along its token axis (Jet-RL explainers, "Schema de Quantification" / "Passage Arriere": dY
 * is quantized for DGrad and for WGrad; X for the forward and for WGrad): 4 bytes of codes written per
 * 2 bytes read, instead of reading the matrix twice.
 * src [rows][cols] -> dst_codes [rows][cols], dst_scales [cols/128][rows], dst_codes_t [cols][rows],
 * dst_scales_t [rows/128][cols].  rows % 128 == 0 and cols % 128 == 0; all four outputs are required. */
int jetfp8_quantize_dual(const void* src_bf16, int64_t rows, int64_t cols, uint8_t* dst_codes,
                         float* dst_scales, uint8_t* dst_codes_t, float* dst_scales_t, void* stream);

/* WGrad operand from a saved FP8 activation.  The pages keep the activations saved for the backward pass in
 * FP8 (Jet-RL explainers, "Schema de Quantification"); WGrad needs X grouped along the token axis.  This
 * takes the 1x128 codes of X and their scales (the JETFP8_ROWS_1x128 outputs), dequantizes each element as
 * one fp32 product decode(code) * scale, and quantizes those values in 128x1 groups along the rows with the
 * same scale and rounding rules as JETFP8_COLS_128x1_T, codes written transposed.  Reads 1 byte per element
 * instead of the 2 of the bf16 matrix.  Finite codes only (0x7F / 0xFF are E4M3 NaN).
 * codes [rows][cols], scales [cols/128][rows] -> dst_codes_t [cols][rows], dst_scales_t [rows/128][cols].
 * rows % 128 == 0 and cols % 128 == 0. */
int jetfp8_requantize_cols_t(const uint8_t* codes, const float* scales, int64_t rows, int64_t cols,
                             uint8_t* dst_codes_t, float* dst_scales_t, void* stream);

/* Fused RMSNorm -> 1x128 quantization.  The activation quantization is fused with the operator that produces
 * the activation (Jet-RL explainers, "Schema de Quantification"), here the RMSNorm in front of a linear layer:
 *   r[i]    = fp32 nearest to 1 / sqrt(mean_k x[i][k]^2 + eps)      (formed in fp64; see below)
 *   y[i][k] = bf16( fl32( fl32(x[i][k] * r[i]) * weight[k] ) )       (round to nearest even)
 *   dst_codes, dst_scales = the JETFP8_ROWS_1x128 quantization of y, bit for bit.
 * x [rows][cols] bf16, weight [cols] bf16 -> dst_codes [rows][cols], dst_scales [cols/128][rows];
 * optional (NULL = not written): dst_rstd [rows] fp32 (r, for the backward), dst_y_bf16 [rows][cols] (y).
 * r is the correctly rounded value unless the exact value lies within about 2^-47 (relative) of a point
 * where its fp32 rounding changes; there either neighbour may be returned.  cols % 128 == 0 and
 * cols <= 8192 (a row is held in registers); 0 < eps <= FLT_MAX (JETFP8_ERR_VALUE otherwise).
 * Finite inputs whose y overflows bf16 give unspecified codes for that group. */
int jetfp8_rmsnorm_quantize(const void* x_bf16, const void* weight_bf16, int64_t rows, int64_t cols, float eps,
                            uint8_t* dst_codes, float* dst_scales, float* dst_rstd, void* dst_y_bf16, void* stream);

/* Fused SwiGLU -> 1x128 quantization (the activation in front of the down projection, quantized by the
 * operator that produces it; Jet-RL explainers, "Schema de Quantification"):
 *   h[i][j] = bf16 nearest to silu(g) * u = g * u / (1 + exp(-g)) of the exact real value, with
 *             g = gate_up[i][j] (gate: columns 0 .. cols-1) and u = gate_up[i][cols + j] (up: cols .. 2cols-1);
 *   dst_codes, dst_scales = the JETFP8_ROWS_1x128 quantization of h, bit for bit.
 * gate_up [rows][2 cols] bf16 -> dst_codes [rows][cols], dst_scales [cols/128][rows]; optional
 * dst_h_bf16 [rows][cols] (h; NULL = not written).  cols % 128 == 0.  Finite inputs; inputs whose h
 * overflows bf16 give unspecified codes for that group. */
int jetfp8_swiglu_quantize(const void* gate_up_bf16, int64_t rows, int64_t cols, uint8_t* dst_codes,
                           float* dst_scales, void* dst_h_bf16, void* stream);

/* Forward FP8 linear (rollout decode, prefill, training forward).  Jet-RL explainers, "Architecture Centrale":
 * rollout runs the same FP8 linear layers, with the same quantization, as the training forward pass;
 * "Schema de Quantification": activations in 1x128 groups, weights in 128x128 blocks, FP8 GEMM.
 *   Y[m][n] = sum_g xs[g][m] * ws[n/128][g] * sum_{k in g} xq[m][k] * wq[n][k]
 * xq [M][K], xs [K/128][M] (JETFP8_ROWS_1x128 of X); wq [N][K], ws [N/128][K/128]
 * (JETFP8_BLOCKS_128x128 of W); y [M][N] bf16.  K % 128 == 0, N % 128 == 0, any M >= 1. */
int jetfp8_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws,
                    void* y_bf16, int64_t M, int64_t N, int64_t K, void* stream);

/* Forward FP8 linear for rollout decode over weights in the fragment order of JETFP8_BLOCKS_128x128_FRAG: the
 * same operation, and bitwise the same result, as jetfp8_gemm_fwd on the row-major codes.  Jet-RL explainers,
 * "Enonce du Probleme": rollout takes over 70 % of RL training time; at decode token counts the GEMM streams the
 * FP8 weights once per step, and this layout lets every weight load read whole 128-byte lines.
 * xq [M][K], xs [K/128][M]; wq_frag (N * K bytes, fragment order), ws [N/128][K/128]; y [M][N] bf16.
 * K % 128 == 0, N % 128 == 0, 1 <= M <= 64 and (K / 128) * M <= 8192 (JETFP8_ERR_SHAPE otherwise). */
int jetfp8_gemm_fwd_frag(const uint8_t* xq, const float* xs, const uint8_t* wq_frag, const float* ws,
                         void* y_bf16, int64_t M, int64_t N, int64_t K, void* stream);

/* DGrad FP8 GEMM (Jet-RL explainers, "Schema de Quantification", backward-pass items: gradients between
 * operators stay BF16, and the DGrad GEMM runs in FP8 with the gradient quantized on entry):
 *   dX[m][k] = sum_g dys[g][m] * ws[g][k/128] * sum_{n in g} dyq[m][n] * wqT[k][n]
 * dyq [M][N], dys [N/128][M] (JETFP8_ROWS_1x128 of dY); wqT [K][N] (the transposed block codes of W
 * from JETFP8_BLOCKS_128x128), ws [N/128][K/128] (the forward block scales, unchanged);
 * dx [M][K] bf16.  N % 128 == 0, K % 128 == 0, any M >= 1. */
int jetfp8_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wqT, const float* ws,
                      void* dx_bf16, int64_t M, int64_t N, int64_t K, void* stream);

/* WGrad FP8 GEMM.  Jet-RL explainers, "Schema de Quantification" / "Esquema de Quantizacao": the weight
 * gradient GEMM runs in FP8 with the "1x128 and 128x1" configuration, read as both operands grouped along the
 * token axis, which is the contraction axis; gradients reach it in BF16 and are quantized on entry:
 *   dW[n][k] = sum_g dysT[g][n] * xsT[g][k] * sum_{m in g} dyqT[n][m] * xqT[k][m]
 * dyqT [N][M], dysT [M/128][N] (JETFP8_COLS_128x1_T of dY); xqT [K][M], xsT [M/128][K]
 * (JETFP8_COLS_128x1_T of X); dw [N][K] bf16, overwritten.  M % 128 == 0, N % 128 == 0,
 * K % 128 == 0. */
int jetfp8_gemm_wgrad(const uint8_t* dyqT, const float* dysT, const uint8_t* xqT, const float* xsT,
                      void* dw_bf16, int64_t M, int64_t N, int64_t K, void* stream);

/* Static, NUL-terminated description of a status code (never NULL). */
const char* jetfp8_status_string(int status);

/* Library version, major*10000 + minor*100 + patch. */
int jetfp8_version(void);

#ifdef __cplusplus
}
#endif

#endif /* JETFP8_H */
