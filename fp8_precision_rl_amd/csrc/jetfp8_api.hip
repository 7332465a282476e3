// C ABI of libjetfp8: host-side validation, then kernel launches on the caller's stream.
// Validation touches no HIP API, so every error path can be exercised without a GPU.
#include <float.h>
#include <stdint.h>

#include "../../include/jetfp8.h"
#include "jetfp8_launch.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;

bool aligned16(const void* p) { return (reinterpret_cast<uintptr_t>(p) & 15u) == 0; }
bool dim_ok(int64_t d) { return d >= 1 && d < kMaxDim; }
int hip_status(hipError_t e) { return e == hipSuccess ? JETFP8_OK : JETFP8_ERR_HIP; }

// Shared checks of the three GEMMs: pointers, alignment, dims, and the axes that must be multiples of 128.
int check_gemm(const void* a, const void* as, const void* b, const void* bs, const void* out, int64_t d0,
               int64_t d1, int64_t d2, bool d0_grouped) {
    if (!a || !as || !b || !bs || !out) return JETFP8_ERR_NULL;
    if (!dim_ok(d0) || !dim_ok(d1) || !dim_ok(d2)) return JETFP8_ERR_SHAPE;
    if (d1 % 128 || d2 % 128 || (d0_grouped && d0 % 128)) return JETFP8_ERR_SHAPE;
    if (!aligned16(a) || !aligned16(as) || !aligned16(b) || !aligned16(bs) || !aligned16(out)) return JETFP8_ERR_ALIGN;
    return JETFP8_OK;
}

// 32-bit offset limits of the GEMM kernels (I rows and J rows of the two operands, contraction Kc): a
// block's 256-row operand band and each scale array must stay below 2^31 bytes.
int check_gemm_extent(int64_t I, int64_t J, int64_t Kc) {
    const int64_t G = Kc / 128;
    if (256 * Kc > jetfp8::kMaxGemmBand || G * I * 4 > jetfp8::kMaxGemmBand || G * J * 4 > jetfp8::kMaxGemmBand)
        return JETFP8_ERR_SHAPE;
    return JETFP8_OK;
}

}  // namespace

extern "C" {

int jetfp8_version(void) { return 302; }

const char* jetfp8_status_string(int status) {
    switch (status) {
        case JETFP8_OK: return "ok";
        case JETFP8_ERR_NULL: return "a required pointer is NULL";
        case JETFP8_ERR_SHAPE: return "bad shape: a dimension is < 1 or >= 2^31, or a grouped/contraction axis is not a multiple of 128";
        case JETFP8_ERR_ALIGN: return "a pointer is not 16-byte aligned";
        case JETFP8_ERR_MODE: return "unknown grouping mode, or a transposed-code output given for a mode without one";
        case JETFP8_ERR_HIP: return "the HIP runtime rejected a kernel launch";
        case JETFP8_ERR_VALUE: return "a scalar argument is outside its domain";
        default: return "unknown status";
    }
}

int jetfp8_quantize(const void* src_bf16, int64_t rows, int64_t cols, int mode, uint8_t* dst_codes,
                    float* dst_scales, uint8_t* dst_codes_t, void* stream) {
    if (mode != JETFP8_ROWS_1x128 && mode != JETFP8_COLS_128x1_T && mode != JETFP8_BLOCKS_128x128 &&
        mode != JETFP8_BLOCKS_128x128_FRAG)
        return JETFP8_ERR_MODE;
    if (dst_codes_t && mode != JETFP8_BLOCKS_128x128 && mode != JETFP8_BLOCKS_128x128_FRAG) return JETFP8_ERR_MODE;
    if (!src_bf16 || !dst_codes || !dst_scales) return JETFP8_ERR_NULL;
    if (!dim_ok(rows) || !dim_ok(cols)) return JETFP8_ERR_SHAPE;
    switch (mode) {
        case JETFP8_ROWS_1x128: if (cols % 128) return JETFP8_ERR_SHAPE; break;
        case JETFP8_COLS_128x1_T: if (rows % 128 || cols % 64) return JETFP8_ERR_SHAPE; break;
        default: if (rows % 128 || cols % 128) return JETFP8_ERR_SHAPE; break;
    }
    const bool fits = mode == JETFP8_ROWS_1x128 ? jetfp8::quant_rows_fits(rows, cols)
                      : mode == JETFP8_COLS_128x1_T ? jetfp8::quant_cols_t_fits(rows, cols)
                                                    : jetfp8::quant_blocks_fits(rows, cols);
    if (!fits) return JETFP8_ERR_SHAPE;
    if (!aligned16(src_bf16) || !aligned16(dst_codes) || !aligned16(dst_scales) ||
        (dst_codes_t && !aligned16(dst_codes_t)))
        return JETFP8_ERR_ALIGN;
    hipStream_t st = static_cast<hipStream_t>(stream);
    const uint16_t* x = static_cast<const uint16_t*>(src_bf16);
    switch (mode) {
        case JETFP8_ROWS_1x128: return hip_status(jetfp8::launch_quant_rows(x, rows, cols, dst_codes, dst_scales, st));
        case JETFP8_COLS_128x1_T: return hip_status(jetfp8::launch_quant_cols_t(x, rows, cols, dst_codes, dst_scales, st));
        default: return hip_status(jetfp8::launch_quant_blocks(x, rows, cols, dst_codes, dst_scales, dst_codes_t,
                                                               mode == JETFP8_BLOCKS_128x128_FRAG, st));
    }
}

int jetfp8_quantize_dual(const void* src_bf16, int64_t rows, int64_t cols, uint8_t* dst_codes, float* dst_scales,
                         uint8_t* dst_codes_t, float* dst_scales_t, void* stream) {
    if (!src_bf16 || !dst_codes || !dst_scales || !dst_codes_t || !dst_scales_t) return JETFP8_ERR_NULL;
    if (!dim_ok(rows) || !dim_ok(cols) || rows % 128 || cols % 128) return JETFP8_ERR_SHAPE;
    if (!jetfp8::quant_dual_fits(rows, cols)) return JETFP8_ERR_SHAPE;
    if (!aligned16(src_bf16) || !aligned16(dst_codes) || !aligned16(dst_scales) || !aligned16(dst_codes_t) ||
        !aligned16(dst_scales_t))
        return JETFP8_ERR_ALIGN;
    return hip_status(jetfp8::launch_quant_dual(static_cast<const uint16_t*>(src_bf16), rows, cols, dst_codes,
                                                dst_scales, dst_codes_t, dst_scales_t,
                                                static_cast<hipStream_t>(stream)));
}

int jetfp8_requantize_cols_t(const uint8_t* codes, const float* scales, int64_t rows, int64_t cols,
                             uint8_t* dst_codes_t, float* dst_scales_t, void* stream) {
    if (!codes || !scales || !dst_codes_t || !dst_scales_t) return JETFP8_ERR_NULL;
    if (!dim_ok(rows) || !dim_ok(cols) || rows % 128 || cols % 128) return JETFP8_ERR_SHAPE;
    if (!jetfp8::quant_requant_cols_fits(rows, cols)) return JETFP8_ERR_SHAPE;
    if (!aligned16(codes) || !aligned16(scales) || !aligned16(dst_codes_t) || !aligned16(dst_scales_t))
        return JETFP8_ERR_ALIGN;
    return hip_status(jetfp8::launch_quant_requant_cols(codes, scales, rows, cols, dst_codes_t, dst_scales_t,
                                                        static_cast<hipStream_t>(stream)));
}

int jetfp8_rmsnorm_quantize(const void* x_bf16, const void* weight_bf16, int64_t rows, int64_t cols, float eps,
                            uint8_t* dst_codes, float* dst_scales, float* dst_rstd, void* dst_y_bf16, void* stream) {
    if (!x_bf16 || !weight_bf16 || !dst_codes || !dst_scales) return JETFP8_ERR_NULL;
    if (!dim_ok(rows) || !dim_ok(cols) || cols % 128 || cols > jetfp8::kRmsNormMaxCols) return JETFP8_ERR_SHAPE;
    if (!(eps > 0.0f && eps <= FLT_MAX)) return JETFP8_ERR_VALUE;
    if (!aligned16(x_bf16) || !aligned16(weight_bf16) || !aligned16(dst_codes) || !aligned16(dst_scales) ||
        (dst_rstd && !aligned16(dst_rstd)) || (dst_y_bf16 && !aligned16(dst_y_bf16)))
        return JETFP8_ERR_ALIGN;
    return hip_status(jetfp8::launch_rmsnorm_quant(static_cast<const uint16_t*>(x_bf16),
                                                   static_cast<const uint16_t*>(weight_bf16), rows, cols, eps,
                                                   dst_codes, dst_scales, dst_rstd, static_cast<uint16_t*>(dst_y_bf16),
                                                   static_cast<hipStream_t>(stream)));
}

int jetfp8_swiglu_quantize(const void* gate_up_bf16, int64_t rows, int64_t cols, uint8_t* dst_codes,
                           float* dst_scales, void* dst_h_bf16, void* stream) {
    if (!gate_up_bf16 || !dst_codes || !dst_scales) return JETFP8_ERR_NULL;
    if (!dim_ok(rows) || !dim_ok(cols) || !dim_ok(2 * cols) || cols % 128) return JETFP8_ERR_SHAPE;
    if (!jetfp8::swiglu_quant_fits(rows, cols)) return JETFP8_ERR_SHAPE;
    if (!aligned16(gate_up_bf16) || !aligned16(dst_codes) || !aligned16(dst_scales) ||
        (dst_h_bf16 && !aligned16(dst_h_bf16)))
        return JETFP8_ERR_ALIGN;
    return hip_status(jetfp8::launch_swiglu_quant(static_cast<const uint16_t*>(gate_up_bf16), rows, cols, dst_codes,
                                                  dst_scales, static_cast<uint16_t*>(dst_h_bf16),
                                                  static_cast<hipStream_t>(stream)));
}

int jetfp8_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, void* y_bf16, int64_t M,
                    int64_t N, int64_t K, void* stream) {
    int rc = check_gemm(xq, xs, wq, ws, y_bf16, M, N, K, false);
    if (rc == JETFP8_OK) rc = check_gemm_extent(M, N, K);
    if (rc != JETFP8_OK) return rc;
    return hip_status(jetfp8::launch_gemm_block_scaled_b(xq, xs, wq, ws, static_cast<uint16_t*>(y_bf16), M, N, K,
                                                         K / 128, 1, static_cast<hipStream_t>(stream)));
}

int jetfp8_gemm_fwd_frag(const uint8_t* xq, const float* xs, const uint8_t* wq_frag, const float* ws, void* y_bf16,
                         int64_t M, int64_t N, int64_t K, void* stream) {
    int rc = check_gemm(xq, xs, wq_frag, ws, y_bf16, M, N, K, false);
    if (rc == JETFP8_OK) rc = check_gemm_extent(M, N, K);
    if (rc != JETFP8_OK) return rc;
    if (!jetfp8::gemm_fwd_frag_fits(M, K)) return JETFP8_ERR_SHAPE;
    return hip_status(jetfp8::launch_gemm_fwd_frag(xq, xs, wq_frag, ws, static_cast<uint16_t*>(y_bf16), M, N, K,
                                                   static_cast<hipStream_t>(stream)));
}

int jetfp8_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wqT, const float* ws, void* dx_bf16,
                      int64_t M, int64_t N, int64_t K, void* stream) {
    int rc = check_gemm(dyq, dys, wqT, ws, dx_bf16, M, N, K, false);
    if (rc == JETFP8_OK) rc = check_gemm_extent(M, K, N);
    if (rc != JETFP8_OK) return rc;
    return hip_status(jetfp8::launch_gemm_block_scaled_b(dyq, dys, wqT, ws, static_cast<uint16_t*>(dx_bf16), M, K, N,
                                                         1, K / 128, static_cast<hipStream_t>(stream)));
}

int jetfp8_gemm_wgrad(const uint8_t* dyqT, const float* dysT, const uint8_t* xqT, const float* xsT, void* dw_bf16,
                      int64_t M, int64_t N, int64_t K, void* stream) {
    int rc = check_gemm(dyqT, dysT, xqT, xsT, dw_bf16, M, N, K, true);
    if (rc == JETFP8_OK) rc = check_gemm_extent(N, K, M);
    if (rc != JETFP8_OK) return rc;
    return hip_status(jetfp8::launch_gemm_row_scaled_b(dyqT, dysT, xqT, xsT, static_cast<uint16_t*>(dw_bf16), N, K, M,
                                                       static_cast<hipStream_t>(stream)));
}

}  // extern "C"
