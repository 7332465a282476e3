/*
 * jetfp8_oracle.c -- plain, slow CPU oracle for the FP8 group-quantize + block-scaled GEMM path.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test suite, the smoke check and the benchmark's CPU-baseline
 * leg may load this library.  The product path (the HIP library) never calls it, shares no code,
 * header, table or helper with it, and must fail loudly when its own extension is missing.
 *
 * What it computes follows the Jet-RL explainers ("Jet-RL: Enabling On-Policy FP8 Reinforcement
 * Learning with Unified Training and Rollout Precision Flow", gist.science fr/pt pages), section
 * "Schema de Quantification" / "Esquema de Quantizacao":
 *   - activations are quantized per 1x128 group, weights per 128x128 block;
 *   - gradients between operators stay BF16; DGrad and WGrad run as FP8 GEMMs (the pt page; the fr
 *     page's "FP16" is read as a slip, the title and the rest of both pages say FP8);
 *   - WGrad uses "1x128 and 128x1" groupings: both of its operands are grouped along the token axis,
 *     which is its contraction axis.
 * The pages give neither the FP8 sub-format nor the scale rule nor the rounding; the readings used here
 * (OCP E4M3, scale = amax/448 in fp32, round to nearest even, saturate at 448, fp32 accumulation per
 * 128-wide group, bf16 output) are listed with each function.
 *
 * Plain loops only: no SIMD intrinsics, no BLAS, no blocking or reordering beyond what the definition
 * states.  Rows may be split across POSIX threads; each output is computed by one thread in the stated
 * order, so the thread count never changes a bit.
 *
 * Parity status (pins live in tests/, marked "not gpu"):
 *   e4m3 decode / encode ....... pinned: all 256 codes, all midpoints, saturation.
 *   bf16 widen / narrow ........ pinned: exhaustive widen, RNE ties, comparison with numpy rounding.
 *   quantizers ................. pinned: hand-computed groups (tests/golden), exact-rational brute force,
 *                                invariants (max element -> +-448, 2^k scale equivariance, sign symmetry).
 *   requantize from FP8 ........ pinned: with power-of-two saved scales x' is a bf16 value and the result
 *                                equals the bf16 128x1 quantizer's; 2^k scale equivariance; sign symmetry.
 *   GEMM, exact group sums ..... pinned: fp64 brute force, K=128 closed form, lossless special case,
 *                                transpose and dgrad identities.
 *   GEMM, matrix-core group sums (JO_GROUPSUM_MFMA) ..... a model of the FP8 matrix instruction's internal
 *                                alignment, which no page describes.  The code is pinned to the stated model
 *                                by hand-derived group sums (tests/golden/group_sums.txt) that builds with
 *                                each plausible model mistake planted in this file fail.  Whether the
 *                                hardware follows the model is measured, not pinned: bit for bit on LLM-like
 *                                and heavy-tailed groups, not on adversarial ones (tests/
 *                                test_gpu_groupsum_model.py).
 *   GEMM accumulation sequence . pinned: exact-rational evaluation of constructed two-group outputs that a
 *                                multiply-then-add, descending group order or a folded row scale would change.
 */
#include <math.h>
#include <pthread.h>
#include <stdint.h>
#include <stdlib.h>
#include <string.h>

/* ------------------------------------------------------------------------------------------------
 * C1.  OCP FP8 E4M3 ("FN": bias 7, no infinities, NaN = S.1111.111, largest finite 448).
 * The pages name FP8 only; E4M3 for every tensor is the reading taken (no E5M2 anywhere).
 * ---------------------------------------------------------------------------------------------- */

/* Value of a code, straight from its bit fields. */
double jo_e4m3_decode(uint8_t c) {
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    double v;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        v = ldexp((double)m, -9);                  /* subnormal: m * 2^-9 */
    else
        v = ldexp(1.0 + (double)m / 8.0, e - 7);   /* normal: (1 + m/8) * 2^(e-7) */
    return s ? -v : v;
}

/* The 127 non-negative finite values in code order 0x00..0x7E (ascending). */
static double g_e4m3_pos[127];
static int g_e4m3_ready = 0;

static void e4m3_table_init(void) {
    if (g_e4m3_ready) return;
    for (int c = 0; c < 127; ++c) g_e4m3_pos[c] = jo_e4m3_decode((uint8_t)c);
    g_e4m3_ready = 1;
}

/* Round a real number to E4M3: nearest representable magnitude, ties to the even code
 * (even code <=> even mantissa field, i.e. IEEE round-half-even), magnitudes beyond 448 saturate to
 * 448 (no NaN is ever produced).  The sign is kept, so a negative value that rounds to zero gives 0x80.
 * Written as a search over the table of values rather than as bit manipulation. */
uint8_t jo_e4m3_encode(double v) {
    e4m3_table_init();
    int neg = signbit(v) ? 1 : 0;
    double a = fabs(v);
    if (a > 448.0) a = 448.0;
    /* largest code whose value is <= a */
    int lo = 0, hi = 126;
    while (lo < hi) {
        int mid = (lo + hi + 1) / 2;
        if (g_e4m3_pos[mid] <= a) lo = mid; else hi = mid - 1;
    }
    int c = lo;
    if (c < 126 && g_e4m3_pos[c] != a) {
        double below = a - g_e4m3_pos[c], above = g_e4m3_pos[c + 1] - a;
        if (above < below || (above == below && (c & 1))) c = c + 1;
    }
    return (uint8_t)(c | (neg << 7));
}

/* ------------------------------------------------------------------------------------------------
 * C2.  bf16 <-> fp32.  Widening is exact.  Narrowing picks the nearer of the two bf16 neighbours,
 * ties to the even bf16 mantissa.  Inputs are finite by contract.
 * ---------------------------------------------------------------------------------------------- */
float jo_bf16_to_f32(uint16_t b) {
    uint32_t u = (uint32_t)b << 16;
    float f;
    memcpy(&f, &u, 4);
    return f;
}

uint16_t jo_f32_to_bf16(float f) {
    uint32_t u;
    memcpy(&u, &f, 4);
    uint32_t toward0 = u & 0xFFFF0000u;          /* magnitude truncated to bf16 */
    if (toward0 == u) return (uint16_t)(u >> 16);
    uint32_t away = toward0 + 0x10000u;          /* next bf16 away from zero */
    float f0, f1;
    memcpy(&f0, &toward0, 4);
    memcpy(&f1, &away, 4);
    /* IEEE rounding with an unbounded exponent, then overflow: past the largest bf16 the next
     * neighbour is 2^128, which becomes infinity. */
    double v1 = isinf(f1) ? copysign(ldexp(1.0, 128), (double)f) : (double)f1;
    double d0 = fabs((double)f - (double)f0), d1 = fabs(v1 - (double)f);
    uint32_t pick;
    if (d0 < d1) pick = toward0;
    else if (d1 < d0) pick = away;
    else pick = ((toward0 >> 16) & 1) ? away : toward0;  /* tie: even mantissa */
    return (uint16_t)(pick >> 16);
}

/* ------------------------------------------------------------------------------------------------
 * C3.  One quantization group: n bf16 values that share one scale.
 *   a = max |x|                        (exact in fp32)
 *   s = fl32(a / 448)                  (IEEE fp32 division, round to nearest even)
 *   s == 0  -> every code is a signed zero (0x00 / 0x80), no NaN
 *   else q  = E4M3(x / s) with x / s the exact quotient.
 * The quotient is formed in fp64: an E4M3 rounding midpoint has at most 5 significant bits, so a
 * quotient of a bf16 value by an fp32 value either equals a midpoint exactly or lies at a relative
 * distance well above 2^-53 from it; the fp64 quotient therefore rounds to the same E4M3 code as the
 * exact one.  ("No calibration", Jet-RL explainers, "Comment ca marche": scales are taken from each
 * tensor on every call.)
 * ---------------------------------------------------------------------------------------------- */
static float group_scale(const float* x, int64_t n, int64_t stride) {
    float a = 0.0f;
    for (int64_t i = 0; i < n; ++i) {
        float v = fabsf(x[i * stride]);
        if (v > a) a = v;
    }
    return a / 448.0f;
}

static uint8_t code_of(float x, float s) {
    if (s == 0.0f) return signbit(x) ? 0x80 : 0x00;
    return jo_e4m3_encode((double)x / (double)s);
}

/* code of a single bf16 value x inside a group whose amax is a (both bf16 bit patterns) */
uint8_t jo_code_for(uint16_t x_bits, uint16_t amax_bits) {
    float a = fabsf(jo_bf16_to_f32(amax_bits));
    return code_of(jo_bf16_to_f32(x_bits), a / 448.0f);
}

/* ------------------------------------------------------------------------------------------------
 * Thread helper: run fn(ctx, i) for i in [0, n) split over nthreads.
 * ---------------------------------------------------------------------------------------------- */
typedef void (*jo_item_fn)(void* ctx, int64_t i);
typedef struct { jo_item_fn fn; void* ctx; int64_t lo, hi; } jo_span;

static void* jo_span_run(void* p) {
    jo_span* s = (jo_span*)p;
    for (int64_t i = s->lo; i < s->hi; ++i) s->fn(s->ctx, i);
    return NULL;
}

static void jo_parallel(int64_t n, int nthreads, jo_item_fn fn, void* ctx) {
    if (nthreads < 1) nthreads = 1;
    if (nthreads > 256) nthreads = 256;
    if (nthreads == 1 || n < 2) {
        for (int64_t i = 0; i < n; ++i) fn(ctx, i);
        return;
    }
    pthread_t th[256];
    jo_span sp[256];
    int started[256];
    for (int t = 0; t < nthreads; ++t) {
        sp[t].fn = fn; sp[t].ctx = ctx;
        sp[t].lo = n * t / nthreads; sp[t].hi = n * (t + 1) / nthreads;
        started[t] = pthread_create(&th[t], NULL, jo_span_run, &sp[t]) == 0;
        if (!started[t]) jo_span_run(&sp[t]);     /* no thread available: do the span here */
    }
    for (int t = 0; t < nthreads; ++t)
        if (started[t]) pthread_join(th[t], NULL);
}

/* ------------------------------------------------------------------------------------------------
 * Quantizers.  Input: bf16 matrix x[R][C] (row-major).  Codes are returned in the logical layout
 * q[r][c] of x; scales are returned group-major, the layout the GEMM reads them in:
 *   rows   (1x128 along C, activations and dY for DGrad):   s[C/128][R]
 *   cols   (128x1 along R, dY and X for WGrad):             s[R/128][C]
 *   blocks (128x128, weights):                              s[R/128][C/128]
 * R, C are multiples of 128 along every grouped axis (callers check).
 * ---------------------------------------------------------------------------------------------- */
typedef struct { const uint16_t* x; int64_t R, C; uint8_t* q; float* s; } jo_qctx;

static void q_rows_item(void* p, int64_t r) {               /* one row: C/128 groups */
    jo_qctx* c = (jo_qctx*)p;
    float buf[128];
    for (int64_t g = 0; g < c->C / 128; ++g) {
        for (int i = 0; i < 128; ++i) buf[i] = jo_bf16_to_f32(c->x[r * c->C + g * 128 + i]);
        float s = group_scale(buf, 128, 1);
        c->s[g * c->R + r] = s;
        for (int i = 0; i < 128; ++i) c->q[r * c->C + g * 128 + i] = code_of(buf[i], s);
    }
}

static void q_cols_item(void* p, int64_t col) {            /* one column: R/128 groups */
    jo_qctx* c = (jo_qctx*)p;
    float buf[128];
    for (int64_t g = 0; g < c->R / 128; ++g) {
        for (int i = 0; i < 128; ++i) buf[i] = jo_bf16_to_f32(c->x[(g * 128 + i) * c->C + col]);
        float s = group_scale(buf, 128, 1);
        c->s[g * c->C + col] = s;
        for (int i = 0; i < 128; ++i) c->q[(g * 128 + i) * c->C + col] = code_of(buf[i], s);
    }
}

static void q_blocks_item(void* p, int64_t rb) {           /* one row of 128x128 blocks */
    jo_qctx* c = (jo_qctx*)p;
    float* buf = (float*)malloc(sizeof(float) * 128 * 128);
    for (int64_t cb = 0; cb < c->C / 128; ++cb) {
        for (int i = 0; i < 128; ++i)
            for (int j = 0; j < 128; ++j)
                buf[i * 128 + j] = jo_bf16_to_f32(c->x[(rb * 128 + i) * c->C + cb * 128 + j]);
        float s = group_scale(buf, 128 * 128, 1);
        c->s[rb * (c->C / 128) + cb] = s;
        for (int i = 0; i < 128; ++i)
            for (int j = 0; j < 128; ++j)
                c->q[(rb * 128 + i) * c->C + cb * 128 + j] = code_of(buf[i * 128 + j], s);
    }
    free(buf);
}

void jo_quantize_rows(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, int nthreads) {
    jo_qctx c = {x, R, C, q, s};
    jo_parallel(R, nthreads, q_rows_item, &c);
}

void jo_quantize_cols(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, int nthreads) {
    jo_qctx c = {x, R, C, q, s};
    jo_parallel(C, nthreads, q_cols_item, &c);
}

void jo_quantize_blocks(const uint16_t* x, int64_t R, int64_t C, uint8_t* q, float* s, int nthreads) {
    jo_qctx c = {x, R, C, q, s};
    jo_parallel(R / 128, nthreads, q_blocks_item, &c);
}

/* ------------------------------------------------------------------------------------------------
 * WGrad operand from a saved FP8 activation.  The pages keep the activations saved for the backward pass
 * in FP8 (Jet-RL explainers, "Schema de Quantification"), while WGrad groups X along the token axis.
 * Reading: the saved 1x128 codes of X, q[R][C] with scales s[C/128][R] (the JETFP8_ROWS_1x128 layout), are
 * dequantized to x' = fl32(decode(q) * s) -- one fp32 product, round to nearest even -- and x' is quantized
 * in 128x1 groups along R exactly as C4 does for a bf16 input: amax exact, s' = fl32(amax / 448), code =
 * nearest E4M3 value to the exact quotient x' / s'.  code_of's fp64 quotient argument holds for an fp32 x'
 * as well: against a midpoint of at most 5 significant bits times a 24-bit s', a 24-bit x' is either an exact
 * midpoint or at a relative distance of about 2^-30 or more, far above the fp64 rounding error.
 * Outputs in the layout of jo_quantize_cols: codes qo[r][c], scales so[R/128][C].
 * ---------------------------------------------------------------------------------------------- */
typedef struct { const uint8_t* q; const float* s; int64_t R, C; uint8_t* qo; float* so; } jo_rqctx;

float jo_dequantize_value(uint8_t code, float scale) {
    const float d = (float)jo_e4m3_decode(code);      /* exact: at most 4 significant bits */
    return d * scale;                                  /* one fp32 product */
}

static void rq_cols_item(void* p, int64_t col) {           /* one column: R/128 groups */
    jo_rqctx* c = (jo_rqctx*)p;
    float buf[128];
    for (int64_t g = 0; g < c->R / 128; ++g) {
        for (int i = 0; i < 128; ++i) {
            const int64_t r = g * 128 + i;
            buf[i] = jo_dequantize_value(c->q[r * c->C + col], c->s[(col / 128) * c->R + r]);
        }
        float sg = group_scale(buf, 128, 1);
        c->so[g * c->C + col] = sg;
        for (int i = 0; i < 128; ++i) c->qo[(g * 128 + i) * c->C + col] = code_of(buf[i], sg);
    }
}

void jo_requantize_cols(const uint8_t* q, const float* s, int64_t R, int64_t C, uint8_t* qo, float* so,
                        int nthreads) {
    jo_rqctx c = {q, s, R, C, qo, so};
    jo_parallel(C, nthreads, rq_cols_item, &c);
}

/* ------------------------------------------------------------------------------------------------
 * Group dot products.  I(c) = decode(c) * 2^9 is an integer with |I| <= 229376, so a product of two
 * codes is an integer multiple of 2^-18 and a 128-term sum is exact in int64.
 *
 * JO_GROUPSUM_EXACT: p = fl32(exact sum)                     -- the plain definition.
 * JO_GROUPSUM_MFMA:  model of an FP8 matrix instruction that forms the 128-term sum in blocks of 8
 *   consecutive terms: inside a block every product is aligned to the largest exponent sum (ea + eb)
 *   of the block and cut toward zero below 2^(emax - 13); the 16 block sums are then added exactly and
 *   rounded once to fp32.  Not from the pages: a stated model of the hardware; see the file header.
 * ---------------------------------------------------------------------------------------------- */
enum { JO_GROUPSUM_EXACT = 0, JO_GROUPSUM_MFMA = 1 };

static int64_t code_int(uint8_t c) {           /* decode(c) * 2^9, exact */
    int s = (c >> 7) & 1, e = (c >> 3) & 15, m = c & 7;
    int64_t v = (e == 0) ? (int64_t)m : (int64_t)(8 + m) << (e - 1);
    return s ? -v : v;
}

static int code_exp(uint8_t c) {               /* unbiased exponent; subnormals use the minimum, -6 */
    int e = (c >> 3) & 15;
    return e == 0 ? -6 : e - 7;
}

static float group_sum_exact(const uint8_t* a, int64_t sa, const uint8_t* b, int64_t sb) {
    int64_t P = 0;
    for (int k = 0; k < 128; ++k) P += code_int(a[k * sa]) * code_int(b[k * sb]);
    return (float)ldexp((double)P, -18);       /* |P| < 2^53: the double is exact, one rounding */
}

static int64_t cut_toward_zero(int64_t x, int sh) {
    if (sh <= 0) return x;
    int64_t m = x < 0 ? -x : x;
    m = (m >> sh) << sh;
    return x < 0 ? -m : m;
}

static float group_sum_mfma(const uint8_t* a, int64_t sa, const uint8_t* b, int64_t sb) {
    int64_t total = 0;
    for (int blk = 0; blk < 16; ++blk) {
        int emax = -1000;
        int64_t prod[8];
        for (int t = 0; t < 8; ++t) {
            uint8_t ca = a[(blk * 8 + t) * sa], cb = b[(blk * 8 + t) * sb];
            prod[t] = code_int(ca) * code_int(cb);
            if (prod[t] != 0 && code_exp(ca) + code_exp(cb) > emax) emax = code_exp(ca) + code_exp(cb);
        }
        /* grid 2^(emax-13) in units of 2^-18 is a shift of emax - 13 + 18 */
        for (int t = 0; t < 8; ++t)
            if (prod[t] != 0) total += cut_toward_zero(prod[t], emax - 13 + 18);
    }
    return (float)ldexp((double)total, -18);
}

typedef float (*jo_gsum_fn)(const uint8_t*, int64_t, const uint8_t*, int64_t);

/* ------------------------------------------------------------------------------------------------
 * C6.  Canonical GEMM: the one fixed per-output sequence (ascending groups, no split of the
 * contraction), fp32 accumulation, bf16 output:
 *     acc = +0
 *     for g = 0, 1, ...:  p = group sum g;  s = fl32(sa * sb);  acc = fma(p, s, acc)
 *     out = bf16(acc)
 * Each GEMM below writes its own index map out in full.
 * ---------------------------------------------------------------------------------------------- */
typedef struct {
    const uint8_t *aq, *bq;
    const float *as, *bs;
    uint16_t* out;
    int64_t M, N, K;
    const int64_t* rows;
    int64_t nrows;
    jo_gsum_fn gsum;
} jo_gctx;

/* Forward:  Y[m][n] = sum_g  sx[g][m] * sw[n/128][g] * sum_{k in g} Xq[m][k] Wq[n][k]
 *   X grouped 1x128 along K, W in 128x128 blocks; both quantized along the contraction axis. */
static void fwd_item(void* p, int64_t r) {
    jo_gctx* c = (jo_gctx*)p;
    int64_t m = c->rows ? c->rows[r] : r, G = c->K / 128;
    for (int64_t n = 0; n < c->N; ++n) {
        float acc = 0.0f;
        for (int64_t g = 0; g < G; ++g) {
            float pg = c->gsum(c->aq + m * c->K + g * 128, 1, c->bq + n * c->K + g * 128, 1);
            float s = c->as[g * c->M + m] * c->bs[(n / 128) * G + g];
            acc = fmaf(pg, s, acc);
        }
        c->out[r * c->N + n] = jo_f32_to_bf16(acc);
    }
}

/* DGrad:  dX[m][k] = sum_g  sdy[g][m] * sw[g][k/128] * sum_{n in g} dYq[m][n] Wq[n][k]
 *   dY grouped 1x128 along N (its contraction axis); W keeps its forward 128x128 block codes and
 *   scales (a block is a block in either orientation), read here down its columns. */
static void dgrad_item(void* p, int64_t r) {
    jo_gctx* c = (jo_gctx*)p;
    int64_t m = c->rows ? c->rows[r] : r, G = c->N / 128, KB = c->K / 128;
    for (int64_t k = 0; k < c->K; ++k) {
        float acc = 0.0f;
        for (int64_t g = 0; g < G; ++g) {
            float pg = c->gsum(c->aq + m * c->N + g * 128, 1, c->bq + (g * 128) * c->K + k, c->K);
            float s = c->as[g * c->M + m] * c->bs[g * KB + k / 128];
            acc = fmaf(pg, s, acc);
        }
        c->out[r * c->K + k] = jo_f32_to_bf16(acc);
    }
}

/* WGrad:  dW[n][k] = sum_g  sdy[g][n] * sx[g][k] * sum_{m in g} dYq[m][n] Xq[m][k]
 *   both operands grouped 128x1 along M (tokens, the contraction axis), re-quantized from bf16. */
static void wgrad_item(void* p, int64_t r) {
    jo_gctx* c = (jo_gctx*)p;
    int64_t n = c->rows ? c->rows[r] : r, G = c->M / 128;
    for (int64_t k = 0; k < c->K; ++k) {
        float acc = 0.0f;
        for (int64_t g = 0; g < G; ++g) {
            float pg = c->gsum(c->aq + (g * 128) * c->N + n, c->N, c->bq + (g * 128) * c->K + k, c->K);
            float s = c->as[g * c->N + n] * c->bs[g * c->K + k];
            acc = fmaf(pg, s, acc);
        }
        c->out[r * c->K + k] = jo_f32_to_bf16(acc);
    }
}

static jo_gsum_fn pick_gsum(int mode) { return mode == JO_GROUPSUM_MFMA ? group_sum_mfma : group_sum_exact; }

/* rows == NULL: all output rows (nrows must then equal the row count); else the listed rows, written
 * densely to out[r][...] in list order. */
void jo_gemm_fwd(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, uint16_t* y,
                 int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, int mode, int nthreads) {
    jo_gctx c = {xq, wq, xs, ws, y, M, N, K, rows, rows ? nrows : M, pick_gsum(mode)};
    jo_parallel(c.nrows, nthreads, fwd_item, &c);
}

void jo_gemm_dgrad(const uint8_t* dyq, const float* dys, const uint8_t* wq, const float* ws, uint16_t* dx,
                   int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, int mode, int nthreads) {
    jo_gctx c = {dyq, wq, dys, ws, dx, M, N, K, rows, rows ? nrows : M, pick_gsum(mode)};
    jo_parallel(c.nrows, nthreads, dgrad_item, &c);
}

/* dyq: codes of dY[M][N] grouped along M (scales dys[M/128][N]); xq: codes of X[M][K] grouped along M
 * (scales xs[M/128][K]).  rows index n (rows of dW). */
void jo_gemm_wgrad(const uint8_t* dyq, const float* dys, const uint8_t* xq, const float* xs, uint16_t* dw,
                   int64_t M, int64_t N, int64_t K, const int64_t* rows, int64_t nrows, int mode, int nthreads) {
    jo_gctx c = {dyq, xq, dys, xs, dw, M, N, K, rows, rows ? nrows : N, pick_gsum(mode)};
    jo_parallel(c.nrows, nthreads, wgrad_item, &c);
}

/* Single group sum, exposed for tests (a, b: 128 codes each). */
float jo_group_sum(const uint8_t* a, const uint8_t* b, int mode) { return pick_gsum(mode)(a, 1, b, 1); }

/* ------------------------------------------------------------------------------------------------
 * C7.  Reference value without the fp32 sequence: sum_g P_g * 2^-18 * sa * sb in fp64 (no bf16
 * rounding).  Used only to check the canonical GEMM against its error bound.
 * ---------------------------------------------------------------------------------------------- */
void jo_gemm_fwd_f64(const uint8_t* xq, const float* xs, const uint8_t* wq, const float* ws, double* y,
                     int64_t M, int64_t N, int64_t K) {
    int64_t G = K / 128;
    for (int64_t m = 0; m < M; ++m)
        for (int64_t n = 0; n < N; ++n) {
            double acc = 0.0;
            for (int64_t g = 0; g < G; ++g) {
                int64_t P = 0;
                for (int k = 0; k < 128; ++k) P += code_int(xq[m * K + g * 128 + k]) * code_int(wq[n * K + g * 128 + k]);
                acc += ldexp((double)P, -18) * ((double)xs[g * M + m] * (double)ws[(n / 128) * G + g]);
            }
            y[m * N + n] = acc;
        }
}
