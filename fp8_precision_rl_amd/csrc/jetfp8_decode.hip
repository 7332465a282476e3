// Small-M schedule of the block-scaled FP8 forward GEMM (rollout decode batches) for gfx950: the same
// per-element operation sequence as the large-M kernels (jetfp8_gemm.hip), so an output row's bits do not depend
// on which schedule computed it (Jet-RL explainers, "Architecture Centrale": the rollout graph is a subgraph of
// the training forward graph with the same quantization).
#include "jetfp8_common.h"
#include "jetfp8_launch.h"
#include "jetfp8_mfma.h"
#include <algorithm>

namespace jetfp8 {

// ---- small-M kernel (rollout decode batches: I <= 16 * RT rows, RT = 1, 2, 4) --------------------------
// The large tiles would leave most of the machine idle and stream each weight row through LDS for a handful
// of output rows, so the decode shape gets its own schedule with the same per-element operation sequence:
//   - the output is cut into slices of 16 columns (16 rows of B) by all I rows; persistent 512-thread blocks
//     take slices b, b + gridDim.x, ... and the operand loads run on across slice boundaries, so the weight
//     stream never drains between slices;
//   - the groups of the contraction are dealt out in chunks of 8, one group per wave: the wave forms the
//     group products of its group with one V_MFMA_F32_16X16X128_F8F6F4 per 16-row tile (B fragment first,
//     C = 0, exactly as the large-M kernels), and parks them in LDS;
//   - after a barrier every wave runs the promotion acc = fma(p, fl32(sa * sb), acc) for its share of the
//     outputs over the chunk's groups in ascending order -- the same chain the large-M kernels run, so every
//     output row is bitwise the same whichever kernel computed it;
//   - operand fragments go straight from global memory into registers, D_AHEAD chunks ahead (2 for RT >= 2;
//     range-checked buffer loads: rows past I and groups past the contraction read as zero and are never
//     promoted); the A-row scales of all groups sit in LDS for the block's lifetime;
//   - the block scales of a chunk's 8 groups come with its operands, one vector load (lane l: group l & 7),
//     and are broadcast with readlane.  Read with scalar loads they held up every chunk: the chunk's barrier
//     waits for LDS traffic with lgkmcnt(0), which also waits for scalar loads in flight (measured: M = 1
//     78 -> 63 us over the four Llama-3-8B linears).
constexpr int D_WAVES = 8, D_THREADS = 64 * D_WAVES, D_AHEAD = 3;
constexpr int D_SA_MAX = 8192;     // A-row scales kept in LDS: (contraction / 128) * rows <= 8192

typedef unsigned int u32x4 __attribute__((ext_vector_type(4)));

// A and As address rows 0 .. I-1 of the call (row m of group g has its scale at As[g * sa_ld + m]), so a call can
// cover a range of a larger batch's rows.
// B layout: FRAG = false, row-major [J][Kc]; FRAG = true, the fragment order written by the block quantizer's
// JETFP8_BLOCKS_128x128_FRAG mode: for each 16-row slice s and group g a 2 KB block at (s * G + g) * 2048 holding
// the 16 B (lo) and then the 16 B (hi) fragment pieces of lanes 0..63, so each of the two loads of a wave's
// fragment reads 1 KB of whole 128-byte lines (row-major, each load touches 16 half-used lines).
template <int RT, bool FRAG>
__global__ __launch_bounds__(D_THREADS) void gemm_decode_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, uint16_t* __restrict__ Cout, int64_t I, int64_t J, int64_t Kc, int64_t sbj,
    int64_t sbg, int64_t sa_ld) {
    // chunks in flight: RT = 2 keeps 2 (82 VGPRs, so two blocks share a CU: measured 4 % faster at 32 rows);
    // RT = 4 keeps 2 to fit its registers; deeper prefetch measured no faster
    constexpr int AHEAD = RT >= 2 ? 2 : D_AHEAD;
    constexpr int PAIRS = RT * 4;                             // (row tile, lane component) pairs of outputs
    constexpr int EPW = (PAIRS + D_WAVES - 1) / D_WAVES;      // pairs per wave in the promotion chain
    constexpr bool ROWC = RT >= 2;                            // row-contiguous A loads (see below)
    __shared__ v4f pbuf[2][D_WAVES][RT][64];
    __shared__ float sa_tab[D_SA_MAX];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int G = (int)(Kc / BK), nchunks = (G + D_WAVES - 1) / D_WAVES;
    const int Ii = (int)I;
    const int slices = (int)(J / 16);
    // chunk stream of this block: slices blockIdx.x, + gridDim.x, ...; nchunks chunks each
    const int nstream = ((slices - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * nchunks;
    auto slice_col = [&](int sc) -> int { return ((int)blockIdx.x + sc * (int)gridDim.x) * 16; };

    // lane l holds row (l & 15) of a 16-row tile, contraction bytes 32 (l >> 4) .. +31 of the group
    const rsrc_t ra = make_rsrc(A, Ii * (int)Kc);
    const int kofs = 32 * (lane >> 4);
    const int vb = FRAG ? 16 * lane : (lane & 15) * (int)Kc + kofs;
    const int vb_hi = FRAG ? vb + 1024 : vb + 16;
    int va[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        va[rt] = ROWC ? (rt * 16 + (lane >> 3)) * (int)Kc + (lane & 7) * 16 : (rt * 16 + (lane & 15)) * (int)Kc + kofs;
    // RT >= 2 (ROWC): the A operand is loaded row-contiguous, each load covering 8 rows x 128 bytes (lane l: row
    // l / 8, 16-byte piece l % 8; the second load rows 8..15), i.e. 8 whole cache lines per instruction instead of
    // 16 half lines, and moved into the matrix instruction's layout (lane t: row t % 16, pieces 2 (t / 16) and
    // 2 (t / 16) + 1) through this wave's own product slot in LDS, one half (8 rows) at a time, the pieces of a row
    // XOR-permuted by the row so the reads spread over the banks.  Measured 10 % faster at 32 rows and 2-4 % at
    // 48-64; at 1-16 rows the direct layout is faster.
    const int wpos = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) << 4);
    const int r8 = lane & 7, q2 = 2 * (lane >> 4);
    const int rpos0 = r8 * 128 + ((q2 ^ r8) << 4), rpos1 = r8 * 128 + (((q2 + 1) ^ r8) << 4);
    const bool hi_rows = (lane & 15) >= 8;

    // promotion-chain ownership: pair q = wave + 8 e -> row tile q >> 2, lane component q & 3
    float acc[EPW];
#pragma unroll
    for (int e = 0; e < EPW; ++e) acc[e] = 0.0f;

    u32x4 wf[AHEAD][2], af[AHEAD][RT][2];
    // block scales of a chunk's 8 groups: lane l holds that of group (l & 7), loaded with the chunk's operands
    // (a vector load, so the per-chunk barrier's LDS wait does not wait for it); range-checked over Bs
    const rsrc_t rbs = make_rsrc(Bs, (int)(J / 128) * G * 4);
    float swf[AHEAD];
    // stream position c -> slice c / nchunks (B rows of that slice only: 16 x Kc bytes), group chunk
    // c % nchunks.  Positions past the block's stream load unconditionally (a conditional load would make
    // the compiler wait for it where the paths join) through an empty descriptor: they read zeros.
    auto load_chunk = [&](int c, u32x4 (&w)[2], u32x4 (&a)[RT][2], float& sw) __attribute__((always_inline)) {
        const int sc = __builtin_amdgcn_readfirstlane(c / nchunks), ch = c - sc * nchunks;
        const bool live = c < nstream;
        {
            const int scc = live ? sc : 0;
            const int gi = min(ch * D_WAVES + (lane & 7), G - 1);
            sw = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(
                rbs, ((slice_col(scc) / 128) * (int)sbj + gi * (int)sbg) * 4, 0, 0));
        }
        const rsrc_t rb = make_rsrc(live ? B + (int64_t)slice_col(sc) * Kc : B, live ? 16 * (int)Kc : 0);
        const int so = (ch * D_WAVES + wave) * BK;
        const int sow = FRAG ? (ch * D_WAVES + wave) * 2048 : so;
        w[0] = __builtin_amdgcn_raw_buffer_load_b128(rb, vb, sow, 0);
        w[1] = __builtin_amdgcn_raw_buffer_load_b128(rb, vb_hi, sow, 0);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            a[rt][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, va[rt], so, 0);
            a[rt][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, va[rt] + (ROWC ? 8 * (int)Kc : 16), so, 0);
        }
    };
    auto store_slice = [&](int sc) __attribute__((always_inline)) {
        const int j0 = slice_col(sc);
        // pair q of lane l is row (q >> 2) * 16 + (l & 15), column j0 + 4 (l >> 4) + (q & 3)
#pragma unroll
        for (int e = 0; e < EPW; ++e) {
            const int q = wave + D_WAVES * e;
            const int m = (q >> 2) * 16 + (lane & 15);
            if (q < PAIRS && m < Ii)
                Cout[(int64_t)m * J + j0 + 4 * (lane >> 4) + (q & 3)] = (uint16_t)f32_to_bf16_rne(acc[e]);
            acc[e] = 0.0f;
        }
    };

    // the A-row scales of every group (the same for all slices) in LDS: sa_tab[g * I + m]; filled before the
    // first operand loads are issued, so waiting for it does not wait for them
    for (int i = t; i < G * Ii; i += D_THREADS) {
        const int g = i / Ii, m = i - g * Ii;
        sa_tab[i] = As[(int64_t)g * sa_ld + m];
    }
#pragma unroll
    for (int k = 0; k < AHEAD; ++k) load_chunk(k, wf[k], af[k], swf[k]);
    // LDS writes done, then every wave is here (a plain barrier: the operand loads stay in flight)
    __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    __builtin_amdgcn_s_barrier();

    auto chunk = [&](int c, u32x4 (&w)[2], u32x4 (&a)[RT][2], float& sw) __attribute__((always_inline)) {
        float sb_cur[D_WAVES];
#pragma unroll
        for (int gi = 0; gi < D_WAVES; ++gi) sb_cur[gi] = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sw), gi));
        const v8i bfrag = (v8i){(int)w[0][0], (int)w[0][1], (int)w[0][2], (int)w[0][3],
                                (int)w[1][0], (int)w[1][1], (int)w[1][2], (int)w[1][3]};
        v4f p[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            u32x4 f0 = a[rt][0], f1 = a[rt][1];
            if (ROWC) {
                // this wave's product slot of two chunks ago: every wave finished reading it before the previous
                // chunk's barrier, and only this wave writes it (1 KB: 64 lanes x 16 bytes)
                uint8_t* slot = reinterpret_cast<uint8_t*>(&pbuf[c & 1][wave][rt][0]);
                u32x4 lo[2], hi[2];
#pragma unroll
                for (int h = 0; h < 2; ++h) {
                    *reinterpret_cast<u32x4*>(slot + wpos) = a[rt][h];
                    lo[h] = *reinterpret_cast<const u32x4*>(slot + rpos0);
                    hi[h] = *reinterpret_cast<const u32x4*>(slot + rpos1);
                }
                f0 = hi_rows ? lo[1] : lo[0];
                f1 = hi_rows ? hi[1] : hi[0];
            }
            const v8i afrag = (v8i){(int)f0[0], (int)f0[1], (int)f0[2], (int)f0[3],
                                    (int)f1[0], (int)f1[1], (int)f1[2], (int)f1[3]};
            p[rt] = mfma_group(bfrag, afrag);
        }
        load_chunk(c + AHEAD, w, a, sw);
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) pbuf[c & 1][wave][rt][lane] = p[rt];
        // this wave's products (and its chain reads of two chunks ago) are in LDS, then every wave is here;
        // a plain barrier, so the operand loads of the next chunks stay in flight
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        __builtin_amdgcn_s_barrier();
        const int ch = c % nchunks;
        // promotion chain over the chunk's groups, ascending.  With 4 row tiles its products and row scales are read
        // first, at clamped indices (a group past the contraction, a row past I or a pair past the tile reads an
        // entry in bounds whose value is not used): read inside the guarded loop, each group's reads waited for
        // the previous group's (measured 4 % faster at 48 and 64 rows; with 1 row tile 6 % slower, so 1 and 2
        // row tiles read in the loop)
        float pv[D_WAVES][EPW], sv[D_WAVES][EPW];
        if constexpr (RT == 4) {
#pragma unroll
            for (int gi = 0; gi < D_WAVES; ++gi) {
                const int gg = min(ch * D_WAVES + gi, G - 1);
#pragma unroll
                for (int e = 0; e < EPW; ++e) {
                    const int q = min(wave + D_WAVES * e, PAIRS - 1);
                    const int m = min((q >> 2) * 16 + (lane & 15), Ii - 1);
                    pv[gi][e] = pbuf[c & 1][gi][q >> 2][lane][q & 3];
                    sv[gi][e] = sa_tab[gg * Ii + m];
                }
            }
        }
#pragma unroll
        for (int gi = 0; gi < D_WAVES; ++gi) {
            if (ch * D_WAVES + gi < G) {
#pragma unroll
                for (int e = 0; e < EPW; ++e) {
                    const int q = wave + D_WAVES * e;
                    const int m = (q >> 2) * 16 + (lane & 15);
                    if (q < PAIRS) {
                        const float p = RT == 4 ? pv[gi][e] : pbuf[c & 1][gi][q >> 2][lane][q & 3];
                        const float sa = m < Ii ? (RT == 4 ? sv[gi][e] : sa_tab[(ch * D_WAVES + gi) * Ii + m]) : 0.0f;
                        acc[e] = fmaf(p, sa * sb_cur[gi], acc[e]);             // s = fl32(sa * sb)
                    }
                }
            }
        }
        if (ch == nchunks - 1) store_slice(c / nchunks);
    };
    int c = 0;
    for (; c + AHEAD <= nstream; c += AHEAD) {
#pragma unroll
        for (int k = 0; k < AHEAD; ++k) chunk(c + k, wf[k], af[k], swf[k]);
    }
#pragma unroll
    for (int k = 0; k < AHEAD; ++k)
        if (c + k < nstream) chunk(c + k, wf[k], af[k], swf[k]);
}

template <int RT, bool FRAG>
static hipError_t launch_decode(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, uint16_t* C,
                                int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg, int64_t sa_ld,
                                hipStream_t st) {
    const int slices = (int)(J / 16);
    // persistent blocks: one per CU, two for RT = 2 (registers and LDS allow it, and it measured faster)
    const int grid = min(slices, (RT == 2 ? 2 : 1) * device_cu_count());
    hipLaunchKernelGGL((gemm_decode_kernel<RT, FRAG>), dim3((unsigned)grid), dim3(D_THREADS), 0, st, A, As, B, Bs, C,
                       I, J, Kc, sbj, sbg, sa_ld);
    return hipGetLastError();
}

// Rows r0 .. r0 + rows - 1 of a call with I rows on the small-M kernel (rows <= 64).
template <bool FRAG>
static hipError_t launch_rows(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, uint16_t* C,
                              int64_t I, int64_t r0, int64_t rows, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg,
                              hipStream_t st) {
    const uint8_t* a = A + r0 * Kc;
    const float* as = As + r0;
    uint16_t* c = C + r0 * J;
    if (rows <= 16) return launch_decode<1, FRAG>(a, as, B, Bs, c, rows, J, Kc, sbj, sbg, I, st);
    if (rows <= 32) return launch_decode<2, FRAG>(a, as, B, Bs, c, rows, J, Kc, sbj, sbg, I, st);
    return launch_decode<4, FRAG>(a, as, B, Bs, c, rows, J, Kc, sbj, sbg, I, st);
}

// ---- small-M schedule for wide outputs over fragment-ordered weights ----------------------------------------
// When there are enough 16-column slices to give every CU several waves (the gate/up projection), each wave owns
// whole slices instead of sharing one slice's groups with its block: it streams its slice's weight fragments
// straight into registers, WIDE_DEPTH groups ahead, multiplies them against the activation fragments, which the
// block keeps in LDS for the whole call (all rows and groups: at most 128 KB), and promotes every product in
// registers in ascending group order.  No barrier or LDS product exchange per group; the per-element sequence is
// the one the other schedules run (acc = fma(p, fl32(sa * sb), acc), groups ascending), so the bits are the
// same.
constexpr int WIDE_DEPTH = 6;                 // weight groups in flight per wave
// weight groups refilled together once consumed: measured against a refill per group on the gate/up projection,
// 24.3 -> 23.2 us at one row and 26.3 -> 25.3 at 32 rows (batches of 2 the same, of 6 slower at 32 rows)
constexpr int WIDE_BATCH = 3;
static_assert(WIDE_DEPTH % WIDE_BATCH == 0, "refill batches tile the prefetch ring");
constexpr int WIDE_A_MAX = 131072;            // activation bytes in LDS: 16 RT rows x contraction
constexpr int WIDE_SA_MAX = 2048;             // activation row scales in LDS: groups x 16 RT
// chunk permutation of a 128-byte activation row in LDS (depends on m & 15: the 16 lanes reading one 16-byte
// column of a fragment hit distinct bank groups)
__device__ __forceinline__ int wide_swz(int m) { return (((m & 7) * 5) & 7) ^ ((m >> 3) & 1); }

#define JETFP8_DEC_LOAD_LDS(r, lds, size, voffset, soffset) \
    __builtin_amdgcn_raw_ptr_buffer_load_lds((r), (lds), (size), (voffset), (soffset), 0, 0)

template <int RT>
__global__ __launch_bounds__(D_THREADS) void gemm_decode_wide_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ Bf,
    const float* __restrict__ Bs, uint16_t* __restrict__ Cout, int I, int J, int Kc) {
    constexpr int MR = 16 * RT;                                  // activation rows kept (zero past I)
    // [g][m][128 bytes], the 16-byte chunks of row m XOR-permuted by swz(m) (the large kernels' layout)
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[WIDE_A_MAX];
    __shared__ float sa_lds[WIDE_SA_MAX];                        // [g][m]
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wpb = (int)(blockDim.x >> 6);
    const int G = Kc / BK, slices = J / 16;
    const int W = (int)gridDim.x * wpb;                          // waves in the grid
    const int gw = wave * (int)gridDim.x + (int)blockIdx.x;      // slices gw, gw + W, ...: consecutive on other CUs

    // this slice's weight fragments: group g at g * 2048 (lane pieces lo, then hi); past the last group the range
    // check (it covers the scalar offset too) reads zeros, so the prefetch runs unconditionally.  The first
    // slice's first groups are requested before the activations are staged.
    u32x4 lo[WIDE_DEPTH], hi[WIDE_DEPTH];
    auto prefetch = [&](int sl, rsrc_t& rb) __attribute__((always_inline)) {
        rb = make_rsrc(Bf + (int64_t)(sl < slices ? sl : 0) * G * 2048, sl < slices ? G * 2048 : 0);
#pragma unroll
        for (int d = 0; d < WIDE_DEPTH; ++d) {
            lo[d] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane, d * 2048, 0);
            hi[d] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane + 1024, d * 2048, 0);
        }
    };
    rsrc_t rb;
    prefetch(gw, rb);

    // activations and their row scales into LDS with direct-to-LDS loads, all in flight at once.  A wave load
    // fills 8 rows of one group (1 KB: lane l at row m0 + l / 8, physical chunk l % 8, which holds the row's chunk
    // (l % 8) ^ wide_swz(m)); rows past I read zeros (range check).  Row scales: 64 consecutive entries of
    // sa_lds [g][m] per load (entries of rows past I hold other scales or zeros: those rows are never stored).
    {
        const rsrc_t ra = make_rsrc(A, I * Kc);
        const rsrc_t rsa = make_rsrc(As, G * I * 4);
        const int nreg = G * (MR / 8);
        for (int q = wave; q < nreg; q += wpb) {
            const int g = q / (MR / 8), m = (q % (MR / 8)) * 8 + (lane >> 3);
            const int vo = m * Kc + g * BK + (((lane & 7) ^ wide_swz(m)) << 4);
            JETFP8_DEC_LOAD_LDS(ra, (lds_void*)(a_lds + q * 1024), 16, vo, 0);
        }
        for (int e0 = wave * 64; e0 < G * MR; e0 += wpb * 64) {
            const int e = e0 + lane, g = e / MR, m = e % MR;
            JETFP8_DEC_LOAD_LDS(rsa, (lds_void*)(sa_lds + e0), 4, (g * I + m) * 4, 0);
        }
    }
    __builtin_amdgcn_s_waitcnt(0);
    __syncthreads();

    const uint32_t rl = lane & 15, cp = 2 * (lane >> 4), sw = (uint32_t)wide_swz((int)rl);
    const int fa0 = (int)(rl * BK + ((cp ^ sw) << 4)), fa1 = (int)(rl * BK + (((cp + 1) ^ sw) << 4));
    for (int sl = gw; sl < slices; sl += W) {
        if (sl != gw) prefetch(sl, rb);
        // block scales of the slice's groups: lane g holds that of group g (G <= 64)
        const rsrc_t rbs = make_rsrc(Bs + (int64_t)(sl >> 3) * G, G * 4);
        const float sbl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, lane * 4, 0, 0));
        v4f acc[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) acc[rt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
        // one group: its product per row tile, promoted in registers
        auto group = [&](int g, int d) __attribute__((always_inline)) {
            const v8i bfrag = (v8i){(int)lo[d][0], (int)lo[d][1], (int)lo[d][2], (int)lo[d][3],
                                    (int)hi[d][0], (int)hi[d][1], (int)hi[d][2], (int)hi[d][3]};
            const float sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sbl), g));
            const uint8_t* ag = a_lds + g * MR * BK;
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const uint4 f0 = *reinterpret_cast<const uint4*>(ag + rt * 16 * BK + fa0);
                const uint4 f1 = *reinterpret_cast<const uint4*>(ag + rt * 16 * BK + fa1);
                const v8i afrag = (v8i){(int)f0.x, (int)f0.y, (int)f0.z, (int)f0.w,
                                        (int)f1.x, (int)f1.y, (int)f1.z, (int)f1.w};
                const v4f p = mfma_group(bfrag, afrag);
                const float s = sa_lds[g * MR + rt * 16 + (int)rl] * sb;      // s = fl32(sa * sb)
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[rt][v] = fmaf(p[v], s, acc[rt][v]);
            }
        };
        // refills in batches of WIDE_BATCH groups (6 KB of the slice in one go)
        auto refill = [&](int g0, int d) __attribute__((always_inline)) {
#pragma unroll
            for (int e = d + 1 - WIDE_BATCH; e <= d; ++e) {
                lo[e] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane, (g0 + e + WIDE_DEPTH) * 2048, 0);
                hi[e] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane + 1024, (g0 + e + WIDE_DEPTH) * 2048, 0);
            }
        };
        // whole steps of WIDE_DEPTH groups without a guard (so the compiler can schedule across their groups), then
        // the guarded last step
        int g0 = 0;
        for (; g0 + WIDE_DEPTH <= G; g0 += WIDE_DEPTH) {
#pragma unroll
            for (int d = 0; d < WIDE_DEPTH; ++d) {
                group(g0 + d, d);
                if ((d + 1) % WIDE_BATCH == 0) refill(g0, d);
            }
        }
        if (g0 < G) {
#pragma unroll
            for (int d = 0; d < WIDE_DEPTH; ++d) {
                if (g0 + d < G) group(g0 + d, d);
                if ((d + 1) % WIDE_BATCH == 0) refill(g0, d);
            }
        }
        // lane l: output row rt * 16 + (l & 15), columns 16 sl + 4 (l >> 4) .. + 3
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            const int m = rt * 16 + (int)rl;
            if (m < I) {
                uint2 w;
                w.x = f32_to_bf16_rne(acc[rt][0]) | (f32_to_bf16_rne(acc[rt][1]) << 16);
                w.y = f32_to_bf16_rne(acc[rt][2]) | (f32_to_bf16_rne(acc[rt][3]) << 16);
                *reinterpret_cast<uint2*>(&Cout[(int64_t)m * J + sl * 16 + 4 * (lane >> 4)]) = w;
            }
        }
    }
}

// ---- wide outputs, activations streamed through LDS in windows -------------------------------------------
// The wide schedule above with the activations staged window by window instead of all at once, so the contraction
// length and the row count (up to 64) are no longer bounded by LDS.  Each wave owns whole slices as above; the
// block steps through windows of WW_WIN groups in lockstep, one barrier per window, with two window buffers in LDS:
// after the barrier that opens window s every wave issues its share of window s + 1's direct-to-LDS loads (codes
// and row scales), then runs window s for its slice.  The weight stream is one sequence over the wave's slices
// (position = round * padded groups + group), refilled WIDE_BATCH groups at a time exactly as above, so a window
// holds the same number of refill loads on every wave (past its last slice a wave refills from an empty
// descriptor): the loads issued after a wave's window loads are exactly the window's refills, which fixes the wait
// that makes them visible.
constexpr int WW_WIN = WIDE_DEPTH;
constexpr int WW_GMAX = 128;
constexpr int WW_REFILLS = 2 * WW_WIN;              // weight loads per window and wave (lo and hi of each group)

template <int RT>
__global__ __launch_bounds__(D_THREADS) void gemm_decode_wwide_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ Bf,
    const float* __restrict__ Bs, uint16_t* __restrict__ Cout, int I, int J, int Kc) {
    constexpr int MR = 16 * RT;
    constexpr int WIN_A = WW_WIN * MR * BK;                          // activation bytes per window
    constexpr int WIN_S = WW_WIN * MR;                               // row scales per window ([g][m])
    __shared__ __attribute__((aligned(16))) uint8_t a_lds[2][WIN_A];
    __shared__ float sa_lds[2][WIN_S + 64];                          // (+ the last load's overhang)
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wpb = (int)(blockDim.x >> 6);
    const int G = Kc / BK, slices = J / 16, nwin = (G + WW_WIN - 1) / WW_WIN, gpad = nwin * WW_WIN;
    const int W = (int)gridDim.x * wpb;                              // waves in the grid
    const int gw = wave * (int)gridDim.x + (int)blockIdx.x;         // slices gw, gw + W, ...
    // slice rounds of the block: those of its wave 0, which has the most
    const int nround = ((int)blockIdx.x < slices) ? (slices - (int)blockIdx.x + W - 1) / W : 0;
    const int nstep = nround * nwin;
    const rsrc_t ra = make_rsrc(A, I * Kc);
    const rsrc_t rsa = make_rsrc(As, G * I * 4);

    // window s's loads into buffer s & 1: WW_WIN groups x MR / 8 regions of 8 rows (lane l: row l / 8, 16-byte
    // piece (l % 8) ^ wide_swz(row)); rows past I read zeros; groups past the contraction read other bytes that are
    // never used.  Row scales: 64 entries [g][m] per load.
    auto stage = [&](int st) __attribute__((always_inline)) {
        const int v = st % nwin, q = st & 1;
        for (int r2 = wave; r2 < WW_WIN * (MR / 8); r2 += wpb) {
            const int gi = r2 / (MR / 8), m = (r2 % (MR / 8)) * 8 + (lane >> 3), g = v * WW_WIN + gi;
            const int vo = m * Kc + g * BK + (((lane & 7) ^ wide_swz(m)) << 4);
            JETFP8_DEC_LOAD_LDS(ra, (lds_void*)(&a_lds[q][0] + r2 * 1024), 16, vo, 0);
        }
        for (int e0 = wave * 64; e0 < WIN_S; e0 += wpb * 64) {
            const int e = e0 + lane, gi = e / MR, m = e % MR, g = v * WW_WIN + gi;
            JETFP8_DEC_LOAD_LDS(rsa, (lds_void*)(&sa_lds[q][0] + e0), 4, (g * I + m) * 4, 0);
        }
    };
    // the weight stream: position p -> slice round p / gpad, group p % gpad
    u32x4 lo[WW_WIN], hi[WW_WIN];
    auto fetch = [&](int p, int d) __attribute__((always_inline)) {
        const int r = p / gpad, g = p - r * gpad, sl = gw + r * W;
        const bool ok = r < nround && sl < slices;
        const rsrc_t rb = make_rsrc(Bf + (int64_t)(ok ? sl : 0) * G * 2048, ok ? G * 2048 : 0);
        lo[d] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane, g * 2048, 0);
        hi[d] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane + 1024, g * 2048, 0);
    };

    if (nstep > 0) stage(0);
#pragma unroll
    for (int d = 0; d < WW_WIN; ++d) fetch(d, d);

    const uint32_t rl = lane & 15, cp = 2 * (lane >> 4), sw = (uint32_t)wide_swz((int)rl);
    const int fa0 = (int)(rl * BK + ((cp ^ sw) << 4)), fa1 = (int)(rl * BK + (((cp + 1) ^ sw) << 4));
    v4f acc[RT];
    float sb0 = 0.0f, sb1 = 0.0f;
    for (int st = 0; st < nstep; ++st) {
        const int r = st / nwin, v = st - r * nwin, sl = gw + r * W;
        const bool live = sl < slices;                               // wave-uniform
        // this wave's loads of window st are done (only the previous window's refills came after them), then
        // every wave's
        __builtin_amdgcn_s_waitcnt((WW_REFILLS & 15) | ((WW_REFILLS >> 4) << 14) | (7 << 4) | (0 << 8));
        asm volatile("" ::: "memory");
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        if (st + 1 < nstep) stage(st + 1);
        if (v == 0) {
            // a new slice: its block scales (lane l: groups l and 64 + l), accumulators cleared
            const rsrc_t rbs = make_rsrc(Bs + (int64_t)((live ? sl : 0) >> 3) * G, live ? G * 4 : 0);
            sb0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, lane * 4, 0, 0));
            sb1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, lane * 4, 256, 0));
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) acc[rt] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
        }
        const uint8_t* aw = &a_lds[st & 1][0];
        const float* sw_ = &sa_lds[st & 1][0];
        const int p0 = r * gpad + v * WW_WIN;
#pragma unroll
        for (int d = 0; d < WW_WIN; ++d) {
            const int g = v * WW_WIN + d;
            if (live && g < G) {
                const v8i bfrag = (v8i){(int)lo[d][0], (int)lo[d][1], (int)lo[d][2], (int)lo[d][3],
                                        (int)hi[d][0], (int)hi[d][1], (int)hi[d][2], (int)hi[d][3]};
                const float sbg = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(g < 64 ? sb0 : sb1), g & 63));
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    const uint8_t* ag = aw + (d * MR + rt * 16) * BK;
                    const uint4 f0 = *reinterpret_cast<const uint4*>(ag + fa0);
                    const uint4 f1 = *reinterpret_cast<const uint4*>(ag + fa1);
                    const v8i afrag = (v8i){(int)f0.x, (int)f0.y, (int)f0.z, (int)f0.w,
                                            (int)f1.x, (int)f1.y, (int)f1.z, (int)f1.w};
                    const v4f pr = mfma_group(bfrag, afrag);
                    const float s = sw_[d * MR + rt * 16 + (int)rl] * sbg;          // s = fl32(sa * sb)
#pragma unroll
                    for (int e = 0; e < 4; ++e) acc[rt][e] = fmaf(pr[e], s, acc[rt][e]);
                }
            }
            if ((d + 1) % WIDE_BATCH == 0) {
#pragma unroll
                for (int e = d + 1 - WIDE_BATCH; e <= d; ++e) fetch(p0 + e + WW_WIN, e);
            }
        }
        if (live && v == nwin - 1) {
            // lane l: output row rt * 16 + (l & 15), columns 16 sl + 4 (l >> 4) .. + 3
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                const int m = rt * 16 + (int)rl;
                if (m < I) {
                    uint2 w2;
                    w2.x = f32_to_bf16_rne(acc[rt][0]) | (f32_to_bf16_rne(acc[rt][1]) << 16);
                    w2.y = f32_to_bf16_rne(acc[rt][2]) | (f32_to_bf16_rne(acc[rt][3]) << 16);
                    *reinterpret_cast<uint2*>(&Cout[(int64_t)m * J + sl * 16 + 4 * (lane >> 4)]) = w2;
                }
            }
        }
        // this wave's reads of the window are done before the next barrier
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
    }
    // every load has landed before the block exits
    __builtin_amdgcn_s_waitcnt(0);
}

// Measured against the slice-sharing kernel (fragment-ordered weights, one process): Llama-3-8B gate/up at 48 and 64
// rows 69.9 -> 30.2 and 75.7 -> 31.4 us; 5120 x 55296 at 32 and 64 rows 86.0 -> 56.7 and 188.9 -> 65.1; 16384 x 16384
// (128 groups) at one row 54.6 -> 49.4.
static bool decode_wwide_fits(int64_t M, int64_t N, int64_t K, int cus) {
    return M <= 64 && K / BK <= WW_GMAX && N / 16 >= 4 * (int64_t)cus;
}

template <int RT>
static hipError_t launch_decode_wwide(const uint8_t* A, const float* As, const uint8_t* Bf, const float* Bs,
                                      uint16_t* C, int64_t M, int64_t N, int64_t K, int cus, hipStream_t st) {
    const int64_t slices = N / 16;
    const int wpb = (int)std::min<int64_t>(D_WAVES, (slices + cus - 1) / cus);
    const int grid = (int)std::min<int64_t>(cus, (slices + wpb - 1) / wpb);
    hipLaunchKernelGGL((gemm_decode_wwide_kernel<RT>), dim3((unsigned)grid), dim3(64 * wpb), 0, st, A, As, Bf, Bs, C,
                       (int)M, (int)N, (int)K);
    return hipGetLastError();
}

// Whether a fragment-ordered forward GEMM takes the wide schedule: at most 32 rows, the activations fit in LDS,
// at most 64 groups, and at least 4 slices per CU.  Measured on the Llama-3-8B gate/up projection (1792 slices):
// 37.7 -> 26.4 us at 32 rows, 30.5 -> 24.8 at 16, 27.5 -> 24.4 at 1; with 1-1.5 slices per CU (O, QKV) it is
// slower than the slice-sharing schedule (O at 32 rows: 8.9 -> 14.7 us).  Prefetch depths 8 and 10 measured
// 1-3 % slower than 6.
static bool decode_wide_fits(int64_t M, int64_t N, int64_t K, int cus) {
    const int64_t mr = M <= 16 ? 16 : 32, G = K / BK;
    return M <= 32 && mr * K <= WIDE_A_MAX && G <= 64 && G * mr <= WIDE_SA_MAX && N / 16 >= 4 * (int64_t)cus;
}

template <int RT>
static hipError_t launch_decode_wide(const uint8_t* A, const float* As, const uint8_t* Bf, const float* Bs,
                                     uint16_t* C, int64_t M, int64_t N, int64_t K, int cus, hipStream_t st) {
    const int64_t slices = N / 16;
    const int wpb = (int)std::min<int64_t>(D_WAVES, (slices + cus - 1) / cus);
    const int grid = (int)std::min<int64_t>(cus, (slices + wpb - 1) / wpb);
    hipLaunchKernelGGL((gemm_decode_wide_kernel<RT>), dim3((unsigned)grid), dim3(64 * wpb), 0, st, A, As, Bf, Bs, C,
                       (int)M, (int)N, (int)K);
    return hipGetLastError();
}

// ---- small-M schedule for narrow outputs over fragment-ordered weights ------------------------------------
// For fewer slices than that (the QKV and O projections), the slice-sharing schedule above keeps too few weight
// bytes in flight.  Here a block takes S adjacent 16-column slices (S = 2 when one slice per block would need
// more blocks than there are CUs) of a contraction of at most 32 groups, dealt out to the 8 waves 4 groups each
// (group 8 i + w to wave w):
//   - each wave requests all its operands at once: the fragment-ordered weights (whole lines) of every slice and
//     one activation fragment per row tile, which serves all S slices;
//   - for 17-32 rows the activation rows are loaded row-contiguous (8 whole lines per load) and moved into the
//     fragment layout through the wave's own LDS: a 2 KB slot per row tile holds both 8-row halves, so each lane
//     reads back only its own 32 bytes (with two slices per block, for LDS room, a 1 KB slot taken one half at a
//     time, as in the slice-sharing schedule; the 2 KB slot measured O 7.4 -> 6.8 us at 32 rows);
//   - the products go to LDS, and after one barrier every thread runs the promotion chain of its outputs (one per
//     slice) over the groups in ascending order: acc = fma(p, fl32(sa * sb), acc).
constexpr int SP_GPW = 4, SP_GMAX = D_WAVES * SP_GPW;

template <int RT, int S>
__global__ __launch_bounds__(D_THREADS) __attribute__((amdgpu_waves_per_eu((RT == 1 && S == 1) ? 3 : 2)))
void gemm_decode_split_kernel(const uint8_t* __restrict__ A, const float* __restrict__ As,
                              const uint8_t* __restrict__ Bf, const float* __restrict__ Bs,
                              uint16_t* __restrict__ Cout, int I, int J, int Kc) {
    constexpr int GPW = SP_GPW, R = SP_GMAX, MR = 16 * RT;
    constexpr bool ROWC = RT >= 2, XFULL = S == 1;
    constexpr int LPR = GPW * (2 * S + 2 * RT);                  // vector loads per wave
    __shared__ v4f pbuf[S][R][RT][64];
    __shared__ float sa_lds[SP_GMAX * MR + 64];                  // [g][m] (+ the last load's overhang)
    __shared__ __attribute__((aligned(16))) uint8_t xbuf[ROWC ? D_WAVES * RT * (XFULL ? 2048 : 1024) : 16];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int sl0 = (int)blockIdx.x * S;
    const int G = Kc / BK;

    // activation row scales into LDS, before any other load (direct-to-LDS, 64 entries per load; entries of rows
    // past I hold other scales or zeros: those rows are never stored)
    {
        const rsrc_t rsa = make_rsrc(As, G * I * 4);
        for (int e0 = wave * 64; e0 < G * MR; e0 += D_THREADS) {
            const int e = e0 + lane, g = e / MR, m = e % MR;
            JETFP8_DEC_LOAD_LDS(rsa, (lds_void*)(sa_lds + e0), 4, (g * I + m) * 4, 0);
        }
    }
    __builtin_amdgcn_sched_barrier(0);
    // block scales of the slices' groups (S <= 2 slices never straddle a 128-row block): lane l holds group l
    const rsrc_t rbs = make_rsrc(Bs + (int64_t)(sl0 >> 3) * G, G * 4);
    const float sbl = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, lane * 4, 0, 0));

    const rsrc_t rb = make_rsrc(Bf + (int64_t)sl0 * G * 2048, S * G * 2048);
    const rsrc_t ra = make_rsrc(A, I * Kc);
    int va[RT];
#pragma unroll
    for (int rt = 0; rt < RT; ++rt)
        va[rt] = ROWC ? (rt * 16 + (lane >> 3)) * Kc + (lane & 7) * 16 : (rt * 16 + (lane & 15)) * Kc + 32 * (lane >> 4);
    // ROWC: lane l loads row l / 8 (the second load rows 8..15), 16-byte piece l % 8; written to the wave's slot
    // with the pieces of a row XOR-permuted by the row, read back as lane t: row t % 16, pieces 2 (t / 16), +1
    const int wpos = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) << 4);
    const int r8 = lane & 7, q2 = 2 * (lane >> 4);
    const int rpos0 = r8 * 128 + ((q2 ^ r8) << 4), rpos1 = r8 * 128 + (((q2 + 1) ^ r8) << 4);
    const bool hi_rows = (lane & 15) >= 8;
    const int fpos0 = (hi_rows ? 1024 : 0) + rpos0, fpos1 = (hi_rows ? 1024 : 0) + rpos1;

    // all operands of the wave's groups (a group past the contraction: weights at an offset past the range, which
    // reads zeros; its activation loads stay in range and are never used)
    u32x4 w[GPW][S][2], a[GPW][RT][2];
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int g = 8 * i + wave;
        const int gc = g < G ? g : 0;
#pragma unroll
        for (int sx = 0; sx < S; ++sx) {
            const int go = g < G ? (sx * G + g) * 2048 : S * G * 2048;
            w[i][sx][0] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane, go, 0);
            w[i][sx][1] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane + 1024, go, 0);
        }
#pragma unroll
        for (int rt = 0; rt < RT; ++rt) {
            a[i][rt][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, va[rt], gc * BK, 0);
            a[i][rt][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, va[rt] + (ROWC ? 8 * Kc : 16), gc * BK, 0);
        }
    }

    // (all of them issued before any product is formed: without the fence the scheduler reuses the first groups'
    // registers for the last group's loads, which then wait for a product)
    __builtin_amdgcn_sched_barrier(0);

    // every product is formed, those of groups past the contraction (zero weights) without being stored: with the
    // products in branches the compiler sinks their operand loads into them, which issues them late
#pragma unroll
    for (int i = 0; i < GPW; ++i) {
        const int g = 8 * i + wave;
        {
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                u32x4 f0 = a[i][rt][0], f1 = a[i][rt][1];
                if (ROWC && XFULL) {
                    uint8_t* slot = xbuf + (wave * RT + rt) * 2048;
                    *reinterpret_cast<u32x4*>(slot + wpos) = a[i][rt][0];
                    *reinterpret_cast<u32x4*>(slot + 1024 + wpos) = a[i][rt][1];
                    f0 = *reinterpret_cast<const u32x4*>(slot + fpos0);
                    f1 = *reinterpret_cast<const u32x4*>(slot + fpos1);
                } else if (ROWC) {
                    uint8_t* slot = xbuf + (wave * RT + rt) * 1024;
                    u32x4 lo[2], hi[2];
#pragma unroll
                    for (int h = 0; h < 2; ++h) {
                        *reinterpret_cast<u32x4*>(slot + wpos) = a[i][rt][h];
                        lo[h] = *reinterpret_cast<const u32x4*>(slot + rpos0);
                        hi[h] = *reinterpret_cast<const u32x4*>(slot + rpos1);
                    }
                    f0 = hi_rows ? lo[1] : lo[0];
                    f1 = hi_rows ? hi[1] : hi[0];
                }
                const v8i afrag = (v8i){(int)f0[0], (int)f0[1], (int)f0[2], (int)f0[3],
                                        (int)f1[0], (int)f1[1], (int)f1[2], (int)f1[3]};
#pragma unroll
                for (int sx = 0; sx < S; ++sx) {
                    const v8i bfrag = (v8i){(int)w[i][sx][0][0], (int)w[i][sx][0][1], (int)w[i][sx][0][2],
                                            (int)w[i][sx][0][3], (int)w[i][sx][1][0], (int)w[i][sx][1][1],
                                            (int)w[i][sx][1][2], (int)w[i][sx][1][3]};
                    const v4f p = mfma_group(bfrag, afrag);
                    if (g < G) pbuf[sx][8 * i + wave][rt][lane] = p;
                }
            }
        }
    }
    // the row-scale loads came first, so with at most this wave's operand loads outstanding they are in LDS (all
    // were consumed above anyway); this wave's products are in LDS; then every wave is here
    __builtin_amdgcn_s_waitcnt((LPR & 15) | ((LPR >> 4) << 14) | (7 << 4));
    __builtin_amdgcn_s_barrier();

    // promotion ownership: thread t < 16 MR holds, in each slice, element t & 3 of lane (t >> 2) & 63 of row tile
    // t >> 8: output row (t >> 8) 16 + ((t >> 2) & 15), column 4 ((t >> 6) & 3) + (t & 3)
    const int ln = (t >> 2) & 63, m = (t >> 8) * 16 + (ln & 15);
    if (t < 16 * MR) {
        // every product and row scale of the chain read first (entries of groups past the contraction are in
        // bounds and unused): in the guarded loop below each group's reads waited for the previous group's
        float pv[S][R], sav[R];
#pragma unroll
        for (int g = 0; g < R; ++g) {
            sav[g] = sa_lds[g * MR + m];
#pragma unroll
            for (int sx = 0; sx < S; ++sx) pv[sx][g] = reinterpret_cast<const float*>(&pbuf[sx][0][0][0])[g * RT * 256 + t];
        }
        float acc[S];
#pragma unroll
        for (int sx = 0; sx < S; ++sx) acc[sx] = 0.0f;
#pragma unroll
        for (int g = 0; g < R; ++g) {
            if (g < G) {
                const float sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sbl), g));
                const float s = sav[g] * sb;                                      // s = fl32(sa * sb)
#pragma unroll
                for (int sx = 0; sx < S; ++sx) acc[sx] = fmaf(pv[sx][g], s, acc[sx]);
            }
        }
        if (m < I) {
#pragma unroll
            for (int sx = 0; sx < S; ++sx)
                Cout[(int64_t)m * J + (sl0 + sx) * 16 + 4 * (ln >> 4) + (t & 3)] = (uint16_t)f32_to_bf16_rne(acc[sx]);
        }
    }
}

// ---- small-M schedule for long contractions over fragment-ordered weights ----------------------------------
// For more than 32 groups (the down projection) the per-slice schedule's rounds pay for their promotion chain on
// the critical path: after each round's barrier every wave promotes before it forms the next round's products.
// Here a block of 16 waves takes one 16-column slice and splits the work by role:
//   - waves 0-7 (producers) take the groups in rounds of 8, group 8 r + w to wave w, request their operands
//     RL_NBUF rounds ahead, form the products (for 17-32 rows through the 2 KB row-contiguous detour above) and park
//     them in LDS;
//   - waves 8-15 (consumers) hold the row scales in LDS and run the promotion chain, one output per thread: after
//     the barrier that closes round r they promote its 8 groups in ascending order, acc = fma(p, fl32(sa * sb),
//     acc), while the producers form round r + 1.
// One barrier per round for both roles; products are double-buffered, and a buffer is refilled only after the
// consumers left it (they pass the next barrier after finishing it).  Measured on the down projection (14336-long
// contraction) against the per-slice schedule's 8-group rounds: 17.3 -> 15.9 us at 32 rows, 16.8 -> 15.5 at 17,
// the same at 1-16 rows.  Blocks this large fit one per CU, which is why the shorter contractions keep the
// per-slice schedule (QKV at 32 rows measured 8.2 -> 9.0 us on it).
constexpr int RL_THREADS = 1024, RL_NBUF = 4, RL_GMAX = 128;

template <int RT>
__global__ __launch_bounds__(RL_THREADS) void gemm_decode_roles_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ Bf,
    const float* __restrict__ Bs, uint16_t* __restrict__ Cout, int I, int J, int Kc) {
    // 4 row tiles (33-64 rows): two rounds in flight and the 1 KB detour slot, for registers and LDS
    constexpr int S = 1, NBUF = RT == 4 ? 2 : RL_NBUF, GMAX = RL_GMAX;
    constexpr bool ROWC = RT >= 2, XFULL = RT <= 2;
    constexpr int R = D_WAVES, MR = 16 * RT;
    constexpr int OPT = (16 * MR + 64 * D_WAVES - 1) / (64 * D_WAVES);   // outputs per consumer thread
    __shared__ v4f pbuf[S][2][R][RT][64];
    __shared__ float sa_lds[GMAX * MR + 64];                     // [g][m] (+ the last load's overhang)
    __shared__ __attribute__((aligned(16))) uint8_t xbuf[ROWC ? D_WAVES * RT * (XFULL ? 2048 : 1024) : 16];
    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int sl0 = (int)blockIdx.x * S;
    const int G = Kc / BK, nr = (G + R - 1) / R;

    if (wave < D_WAVES) {
        // ---- producer ----
        const rsrc_t rb = make_rsrc(Bf + (int64_t)sl0 * G * 2048, S * G * 2048);
        const rsrc_t ra = make_rsrc(A, I * Kc);
        int va[RT];
#pragma unroll
        for (int rt = 0; rt < RT; ++rt)
            va[rt] = ROWC ? (rt * 16 + (lane >> 3)) * Kc + (lane & 7) * 16
                          : (rt * 16 + (lane & 15)) * Kc + 32 * (lane >> 4);
        // ROWC: lane l loads row l / 8 (the second load rows 8..15), 16-byte piece l % 8; written to the wave's
        // slot with the pieces of a row XOR-permuted by the row, read back as lane t: row t % 16, pieces 2 (t / 16),
        // 2 (t / 16) + 1
        const int wpos = (lane >> 3) * 128 + (((lane & 7) ^ (lane >> 3)) << 4);
        const int r8 = lane & 7, q2 = 2 * (lane >> 4);
        const int rpos0 = r8 * 128 + ((q2 ^ r8) << 4), rpos1 = r8 * 128 + (((q2 + 1) ^ r8) << 4);
        const bool hi_rows = (lane & 15) >= 8;
        const int fpos0 = (hi_rows ? 1024 : 0) + rpos0, fpos1 = (hi_rows ? 1024 : 0) + rpos1;

        u32x4 wf[NBUF][S][2], af[NBUF][RT][2];
        // round r's operands (a group past the contraction: weights at an offset past the range, which reads
        // zeros; its activation loads stay in range and are never used)
        auto load_round = [&](int r, u32x4 (&w)[S][2], u32x4 (&a)[RT][2]) __attribute__((always_inline)) {
            const int g = r * R + wave;
            const int gc = g < G ? g : 0;
#pragma unroll
            for (int sx = 0; sx < S; ++sx) {
                const int go = g < G ? (sx * G + g) * 2048 : S * G * 2048;
                w[sx][0] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane, go, 0);
                w[sx][1] = __builtin_amdgcn_raw_buffer_load_b128(rb, 16 * lane + 1024, go, 0);
            }
#pragma unroll
            for (int rt = 0; rt < RT; ++rt) {
                a[rt][0] = __builtin_amdgcn_raw_buffer_load_b128(ra, va[rt], gc * BK, 0);
                a[rt][1] = __builtin_amdgcn_raw_buffer_load_b128(ra, va[rt] + (ROWC ? 8 * Kc : 16), gc * BK, 0);
            }
        };
#pragma unroll
        for (int k = 0; k < NBUF; ++k)
            if (k < nr) load_round(k, wf[k], af[k]);

        auto round = [&](int r, u32x4 (&w)[S][2], u32x4 (&a)[RT][2]) __attribute__((always_inline)) {
            const int g = r * R + wave;
            if (g < G) {
#pragma unroll
                for (int rt = 0; rt < RT; ++rt) {
                    u32x4 f0 = a[rt][0], f1 = a[rt][1];
                    if (ROWC && XFULL) {
                        uint8_t* slot = xbuf + (wave * RT + rt) * 2048;
                        *reinterpret_cast<u32x4*>(slot + wpos) = a[rt][0];
                        *reinterpret_cast<u32x4*>(slot + 1024 + wpos) = a[rt][1];
                        f0 = *reinterpret_cast<const u32x4*>(slot + fpos0);
                        f1 = *reinterpret_cast<const u32x4*>(slot + fpos1);
                    } else if (ROWC) {
                        uint8_t* slot = xbuf + (wave * RT + rt) * 1024;
                        u32x4 lo[2], hi[2];
#pragma unroll
                        for (int h = 0; h < 2; ++h) {
                            *reinterpret_cast<u32x4*>(slot + wpos) = a[rt][h];
                            lo[h] = *reinterpret_cast<const u32x4*>(slot + rpos0);
                            hi[h] = *reinterpret_cast<const u32x4*>(slot + rpos1);
                        }
                        f0 = hi_rows ? lo[1] : lo[0];
                        f1 = hi_rows ? hi[1] : hi[0];
                    }
                    const v8i afrag = (v8i){(int)f0[0], (int)f0[1], (int)f0[2], (int)f0[3],
                                            (int)f1[0], (int)f1[1], (int)f1[2], (int)f1[3]};
#pragma unroll
                    for (int sx = 0; sx < S; ++sx) {
                        const v8i bfrag = (v8i){(int)w[sx][0][0], (int)w[sx][0][1], (int)w[sx][0][2],
                                                (int)w[sx][0][3], (int)w[sx][1][0], (int)w[sx][1][1],
                                                (int)w[sx][1][2], (int)w[sx][1][3]};
                        pbuf[sx][r & 1][wave][rt][lane] = mfma_group(bfrag, afrag);
                    }
                }
            }
            if (r + NBUF < nr) load_round(r + NBUF, w, a);
            // this wave's products are in LDS, then every wave is here (the consumers finished round r - 1,
            // so the buffer round r + 1 will fill is free)
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
            __builtin_amdgcn_s_barrier();
        };
        for (int r = 0; r < nr; r += NBUF) {
#pragma unroll
            for (int k = 0; k < NBUF; ++k)
                if (r + k < nr) round(r + k, wf[k], af[k]);
        }
    } else {
        // ---- consumer ----
        const int tc = t - 64 * D_WAVES, cw = wave - D_WAVES;
        // activation row scales into LDS (direct-to-LDS, 64 entries per load; entries of rows past I hold other
        // scales or zeros: those rows are never stored), block scales of the slices' groups (S <= 2 slices never
        // straddle a 128-row block): lane l holds group l (sb0) and group 64 + l (sb1)
        const rsrc_t rsa = make_rsrc(As, G * I * 4);
        for (int e0 = cw * 64; e0 < G * MR; e0 += 64 * D_WAVES) {
            const int e = e0 + lane, g = e / MR, m = e % MR;
            JETFP8_DEC_LOAD_LDS(rsa, (lds_void*)(sa_lds + e0), 4, (g * I + m) * 4, 0);
        }
        const rsrc_t rbs = make_rsrc(Bs + (int64_t)(sl0 >> 3) * G, G * 4);
        const float sb0 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, lane * 4, 0, 0));
        const float sb1 = __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, lane * 4, 256, 0));
        __builtin_amdgcn_s_waitcnt(0);
        // output ownership: consumer thread tc holds outputs u = tc + 512 h (h < OPT, u < 16 MR): in each slice,
        // element u & 3 of lane (u >> 2) & 63 of row tile u >> 8, i.e. output row (u >> 8) 16 + ((u >> 2) & 15),
        // column 4 ((u >> 6) & 3) + (u & 3)
        float acc[OPT][S];
#pragma unroll
        for (int h = 0; h < OPT; ++h)
#pragma unroll
            for (int sx = 0; sx < S; ++sx) acc[h][sx] = 0.0f;
        for (int r = 0; r < nr; ++r) {
            __builtin_amdgcn_s_barrier();
            const float sbr = r * R < 64 ? sb0 : sb1;             // R divides 64: a round lies in one half
#pragma unroll
            for (int h = 0; h < OPT; ++h) {
                const int u = tc + 64 * D_WAVES * h;
                const int m = (u >> 8) * 16 + ((u >> 2) & 15);
                if (u < 16 * MR) {
                    // the round's products and row scales read first (a group past the contraction is in bounds:
                    // the rounds cover at most RL_GMAX groups, a multiple of the round; its entries are unused)
                    float pv[S][R], sav[R];
#pragma unroll
                    for (int ig = 0; ig < R; ++ig) {
                        sav[ig] = sa_lds[(r * R + ig) * MR + m];
#pragma unroll
                        for (int sx = 0; sx < S; ++sx)
                            pv[sx][ig] = reinterpret_cast<const float*>(&pbuf[sx][r & 1][0][0][0])[ig * RT * 256 + u];
                    }
#pragma unroll
                    for (int ig = 0; ig < R; ++ig) {
                        const int g = r * R + ig;
                        if (g < G) {
                            const float sb = __int_as_float(__builtin_amdgcn_readlane(__float_as_int(sbr), g & 63));
                            const float s = sav[ig] * sb;                         // s = fl32(sa * sb)
#pragma unroll
                            for (int sx = 0; sx < S; ++sx) acc[h][sx] = fmaf(pv[sx][ig], s, acc[h][sx]);
                        }
                    }
                }
            }
            // this round's product reads are done before the next barrier
            __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        }
#pragma unroll
        for (int h = 0; h < OPT; ++h) {
            const int u = tc + 64 * D_WAVES * h;
            const int m = (u >> 8) * 16 + ((u >> 2) & 15);
            if (u < 16 * MR && m < I) {
#pragma unroll
                for (int sx = 0; sx < S; ++sx)
                    Cout[(int64_t)m * J + (sl0 + sx) * 16 + 4 * ((u >> 6) & 3) + (u & 3)] =
                        (uint16_t)f32_to_bf16_rne(acc[h][sx]);
            }
        }
    }
}

// Which small-M schedule a fragment-ordered forward GEMM takes: the wide one when its activations fit in LDS, else
// the windowed wide one for at least 4 slices per CU (up to 64 rows and 128 groups; where both fit the first measured
// faster: gate/up at 32 rows 25.5 against 28.0 us, its waves run unsynchronized), else:
//   - at most 32 rows and 32 groups: the one-round per-slice kernel (with fewer than 4 slices per CU; from 4 per CU
//     on, the wide kernel fits, since the activations of 32 groups fit in LDS);
//   - 33-128 groups (and any contraction at 33-64 rows): the role-split kernel, when its one-block-per-slice rounds
//     stay short: at most one slice per CU, or two for contractions of at least 64 groups or for more than 32 rows
//     (at 48 rows QKV measured 20.9 -> 18.2 us, 4096 x 8192 20.8 -> 18.0); otherwise the slice-sharing kernel,
//     whose persistent blocks stream on across slices.
// Measured against the slice-sharing kernel at 32 rows (fragment-ordered weights, one process): QKV 12.6 -> 8.5 us,
// O 9.0 -> 6.6, down (14336 x 4096) 23.5 -> 15.4, 16384 x 8192 43.3 -> 39.5; but 5120 x 13824 (3.4 slices per CU,
// 40 groups) 24.7 -> 28.6 and 5120 x 27648 45.9 -> 61.8 on the role-split kernel, which is why those do not take it
// (5120 x 13824 keeps the slice-sharing kernel; 5120 x 27648 has enough slices for the windowed wide one).
enum class SmallM { kWide, kWWide, kSplit, kRoles, kShared };
static SmallM decode_schedule(int64_t M, int64_t N, int64_t K, int cus) {
    const int64_t G = K / BK, slices = N / 16;
    if (decode_wide_fits(M, N, K, cus)) return SmallM::kWide;
    if (decode_wwide_fits(M, N, K, cus)) return SmallM::kWWide;
    if (M > 64) return SmallM::kShared;
    if (M <= 32 && G <= SP_GMAX) return SmallM::kSplit;
    if (G <= RL_GMAX && (slices <= cus || (slices <= 2 * (int64_t)cus && (G >= 64 || M > 32)))) return SmallM::kRoles;
    return SmallM::kShared;
}

template <int RT>
static hipError_t launch_decode_split(const uint8_t* A, const float* As, const uint8_t* Bf, const float* Bs,
                                      uint16_t* C, int64_t M, int64_t N, int64_t K, int cus, hipStream_t st) {
    const int slices = (int)(N / 16);
    const int i = (int)M, j = (int)N, kc = (int)K;
    if constexpr (RT == 2) {
        if (slices > cus) {                 // slices is a multiple of 8 (N % 128 == 0)
            hipLaunchKernelGGL((gemm_decode_split_kernel<RT, 2>), dim3((unsigned)(slices / 2)), dim3(D_THREADS), 0, st,
                               A, As, Bf, Bs, C, i, j, kc);
            return hipGetLastError();
        }
    }
    hipLaunchKernelGGL((gemm_decode_split_kernel<RT, 1>), dim3((unsigned)slices), dim3(D_THREADS), 0, st, A, As, Bf,
                       Bs, C, i, j, kc);
    return hipGetLastError();
}

template <int RT>
static hipError_t launch_decode_roles(const uint8_t* A, const float* As, const uint8_t* Bf, const float* Bs,
                                      uint16_t* C, int64_t M, int64_t N, int64_t K, hipStream_t st) {
    hipLaunchKernelGGL((gemm_decode_roles_kernel<RT>), dim3((unsigned)(N / 16)), dim3(RL_THREADS), 0, st, A, As, Bf,
                       Bs, C, (int)M, (int)N, (int)K);
    return hipGetLastError();
}

bool decode_rows_fit(int64_t rows, int64_t Kc) { return rows <= 64 && (Kc / BK) * rows <= D_SA_MAX; }

hipError_t launch_decode_rows(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, uint16_t* C,
                              int64_t I, int64_t r0, int64_t rows, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg,
                              hipStream_t st) {
    return launch_rows<false>(A, As, B, Bs, C, I, r0, rows, J, Kc, sbj, sbg, st);
}

bool gemm_fwd_frag_fits(int64_t M, int64_t K) { return decode_rows_fit(M, K); }

// Forward GEMM over fragment-ordered weights (the small-M kernel only; the caller checks gemm_fwd_frag_fits).
hipError_t launch_gemm_fwd_frag(const uint8_t* xq, const float* xs, const uint8_t* wqf, const float* ws, uint16_t* y,
                                int64_t M, int64_t N, int64_t K, hipStream_t st) {
    const int cus = device_cu_count();
    switch (decode_schedule(M, N, K, cus)) {
    case SmallM::kWide:
        return M <= 16 ? launch_decode_wide<1>(xq, xs, wqf, ws, y, M, N, K, cus, st)
                       : launch_decode_wide<2>(xq, xs, wqf, ws, y, M, N, K, cus, st);
    case SmallM::kWWide:
        return M <= 16 ? launch_decode_wwide<1>(xq, xs, wqf, ws, y, M, N, K, cus, st)
                       : M <= 32 ? launch_decode_wwide<2>(xq, xs, wqf, ws, y, M, N, K, cus, st)
                                 : launch_decode_wwide<4>(xq, xs, wqf, ws, y, M, N, K, cus, st);
    case SmallM::kSplit:
        return M <= 16 ? launch_decode_split<1>(xq, xs, wqf, ws, y, M, N, K, cus, st)
                       : launch_decode_split<2>(xq, xs, wqf, ws, y, M, N, K, cus, st);
    case SmallM::kRoles:
        return M <= 16 ? launch_decode_roles<1>(xq, xs, wqf, ws, y, M, N, K, st)
                       : M <= 32 ? launch_decode_roles<2>(xq, xs, wqf, ws, y, M, N, K, st)
                                 : launch_decode_roles<4>(xq, xs, wqf, ws, y, M, N, K, st);
    case SmallM::kShared:
        break;
    }
    return launch_rows<true>(xq, xs, wqf, ws, y, M, 0, M, N, K, K / BK, 1, st);
}

}  // namespace jetfp8
