/* Host driver that runs every entry point of the CPU oracle (oracle/jetfp8_oracle.c) on small seeded inputs,
 * for a build with AddressSanitizer and UndefinedBehaviorSanitizer (tests/test_oracle_sanitizers.py).  Each
 * buffer is allocated at its exact size, so any read or write past one is reported.  Exits 0 when every call
 * returns; the sanitizers abort the process on the first error. */
#include <math.h>
#include <stdint.h>
#include <stdio.h>
#include <stdlib.h>
#include <string.h>

double jo_e4m3_decode(uint8_t c);
uint8_t jo_e4m3_encode(double v);
float jo_bf16_to_f32(uint16_t b);
uint16_t jo_f32_to_bf16(float f);
uint8_t jo_code_for(uint16_t x_bits, uint16_t amax_bits);
void jo_quantize_rows(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, int nthreads);
void jo_quantize_cols(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, int nthreads);
void jo_quantize_blocks(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, int nthreads);
float jo_dequantize_value(uint8_t code, float scale);
void jo_requantize_cols(const uint8_t* q, const float* s, int64_t R, int64_t C, uint8_t* qo, float* so, int nthreads);
void jo_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, uint16_t* y, int64_t M,
                 int64_t N, int64_t K, const int64_t* rows, int64_t nrows, int mode, int nthreads);
void jo_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq, const float* ws, uint16_t* dx, int64_t M,
                   int64_t N, int64_t K, const int64_t* rows, int64_t nrows, int mode, int nthreads);
void jo_gemm_wgrad(const uint8_t* dyq, const float* dys, const uint8_t* xq, const float* xs, uint16_t* dw, int64_t M,
                   int64_t N, int64_t K, const int64_t* rows, int64_t nrows, int mode, int nthreads);
float jo_group_sum(const uint8_t* a, const uint8_t* b, int mode);
void jo_gemm_fwd_f64(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, double* y, int64_t M,
                     int64_t N, int64_t K);

static uint64_t g_state = 0x9E3779B97F4A7C15ull;
static uint32_t next_u32(void) {                    /* xorshift64*, seeded */
    g_state ^= g_state >> 12;
    g_state ^= g_state << 25;
    g_state ^= g_state >> 27;
    return (uint32_t)((g_state * 0x2545F4914F6CDD1Dull) >> 32);
}

/* a finite bf16 pattern: random sign and fraction, exponent field 0..254 (zero and subnormals included) */
static uint16_t finite_bf16(void) {
    uint32_t r = next_u32();
    uint16_t e = (uint16_t)(r % 255u);
    return (uint16_t)(((r >> 8) & 0x8000u) | (e << 7) | ((r >> 16) & 0x7Fu));
}

static void* xmalloc(size_t n) {
    void* p = malloc(n ? n : 1);
    if (!p) { fprintf(stderr, "out of memory\n"); exit(2); }
    return p;
}

int main(void) {
    /* codec, widen / narrow, one-value quantizer */
    for (int c = 0; c < 256; ++c) {
        double v = jo_e4m3_decode((uint8_t)c);
        if (!isnan(v)) (void)jo_e4m3_encode(v);
    }
    for (uint32_t b = 0; b < 65536; b += 7) (void)jo_f32_to_bf16(jo_bf16_to_f32((uint16_t)b) * 1.0009765625f);
    for (int i = 0; i < 4096; ++i) (void)jo_code_for(finite_bf16(), finite_bf16());

    const int64_t R = 256, C = 384, M = 256, N = 256, K = 384;     /* several groups and blocks each way */
    uint16_t* x = xmalloc(sizeof(uint16_t) * R * C);
    for (int64_t i = 0; i < R * C; ++i) x[i] = finite_bf16();
    for (int64_t k = 0; k < C; ++k) x[5 * C + k] = 0;              /* an all-zero row */
    uint8_t* q = xmalloc(R * C);
    float* s_rows = xmalloc(sizeof(float) * (C / 128) * R);
    float* s_cols = xmalloc(sizeof(float) * (R / 128) * C);
    float* s_blk = xmalloc(sizeof(float) * (R / 128) * (C / 128));
    uint8_t* q2 = xmalloc(R * C);
    for (int t = 1; t <= 5; t += 4) {                                /* one thread, and more threads than rows need */
        jo_quantize_rows(x, R, C, q, s_rows, t);
        jo_quantize_cols(x, R, C, q2, s_cols, t);
        jo_quantize_blocks(x, R, C, q2, s_blk, t);
    }
    jo_quantize_rows(x, 3, 128, q, s_rows, 8);                       /* fewer rows than threads */
    jo_quantize_rows(x, R, C, q, s_rows, 3);
    (void)jo_dequantize_value(q[0], s_rows[0]);
    uint8_t* qo = xmalloc(R * C);
    float* so = xmalloc(sizeof(float) * (R / 128) * C);
    jo_requantize_cols(q, s_rows, R, C, qo, so, 4);

    /* GEMMs: operands from the quantizers, both group-sum modes, all rows and a row list */
    uint16_t* w = xmalloc(sizeof(uint16_t) * N * K);
    for (int64_t i = 0; i < N * K; ++i) w[i] = finite_bf16();
    uint8_t* wq = xmalloc(N * K);
    float* ws = xmalloc(sizeof(float) * (N / 128) * (K / 128));
    jo_quantize_blocks(w, N, K, wq, ws, 2);
    uint8_t* xq = xmalloc(M * K);
    float* xs = xmalloc(sizeof(float) * (K / 128) * M);
    jo_quantize_rows(x, M, K, xq, xs, 2);
    uint16_t* y = xmalloc(sizeof(uint16_t) * M * N);
    const int64_t rows[3] = {M - 1, 0, 7};
    for (int mode = 0; mode < 2; ++mode) {
        jo_gemm_fwd(xq, xs, wq, ws, y, M, N, K, NULL, M, mode, 3);
        jo_gemm_fwd(xq, xs, wq, ws, y, M, N, K, rows, 3, mode, 2);
    }
    /* DGrad: dY [M, N'] with N' = K (the contraction), W [N', K'] = wq read as [K, N] */
    uint8_t* dyq = xmalloc(M * K);
    float* dys = xmalloc(sizeof(float) * (K / 128) * M);
    jo_quantize_rows(x, M, K, dyq, dys, 1);
    uint16_t* dx = xmalloc(sizeof(uint16_t) * M * N);
    uint8_t* wqT = xmalloc(K * N);
    float* wsT = xmalloc(sizeof(float) * (K / 128) * (N / 128));
    for (int64_t n = 0; n < N; ++n)
        for (int64_t k = 0; k < K; ++k) wqT[k * N + n] = wq[n * K + k];
    for (int64_t a = 0; a < N / 128; ++a)
        for (int64_t b = 0; b < K / 128; ++b) wsT[b * (N / 128) + a] = ws[a * (K / 128) + b];
    for (int mode = 0; mode < 2; ++mode) {
        jo_gemm_dgrad(dyq, dys, wqT, wsT, dx, M, K, N, NULL, M, mode, 4);
        jo_gemm_dgrad(dyq, dys, wqT, wsT, dx, M, K, N, rows, 3, mode, 1);
    }
    /* WGrad: both operands grouped along M */
    uint8_t* dyqc = xmalloc(M * N);
    float* dysc = xmalloc(sizeof(float) * (M / 128) * N);
    jo_quantize_cols(w, M, N, dyqc, dysc, 2);                        /* any [M, N] bf16 matrix */
    uint8_t* xqc = xmalloc(M * K);
    float* xsc = xmalloc(sizeof(float) * (M / 128) * K);
    jo_quantize_cols(x, M, K, xqc, xsc, 2);
    uint16_t* dw = xmalloc(sizeof(uint16_t) * N * K);
    const int64_t nrows[2] = {N - 1, 3};
    for (int mode = 0; mode < 2; ++mode) {
        jo_gemm_wgrad(dyqc, dysc, xqc, xsc, dw, M, N, K, NULL, N, mode, 5);
        jo_gemm_wgrad(dyqc, dysc, xqc, xsc, dw, M, N, K, nrows, 2, mode, 1);
    }
    (void)jo_group_sum(xq, wq, 0);
    (void)jo_group_sum(xq, wq, 1);
    double* y64 = xmalloc(sizeof(double) * M * N);
    jo_gemm_fwd_f64(xq, xs, wq, ws, y64, M, N, K);

    free(x); free(q); free(s_rows); free(s_cols); free(s_blk); free(q2); free(qo); free(so); free(w); free(wq);
    free(ws); free(xq); free(xs); free(y); free(dyq); free(dys); free(dx); free(wqT); free(wsT); free(dyqc);
    free(dysc); free(xqc); free(xsc); free(dw); free(y64);
    printf("oracle sanitizer driver: all calls returned\n");
    return 0;
}
