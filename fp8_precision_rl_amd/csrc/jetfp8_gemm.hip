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
// Layout of the work (large-M kernels):
//   - 512 threads = 8 waves (2 per SIMD), block tile 256 x 256, wave tile 128 x 64 (8 x 4 MFMA tiles), so
//     each fragment byte read from LDS feeds 2.7 matrix ops on average (LDS bandwidth is the tight resource);
//   - A and B group tiles and their scales stream global -> LDS with buffer_load ... lds into a 2-stage
//     ring (one group in flight while one is multiplied);
//   - two schedules: gemm_large_kernel interleaves the two waves of each SIMD (one barrier per group; WGrad, and
//     128 x 128 quarter tiles for every GEMM), gemm_pp_kernel runs them in alternating memory and compute phases
//     (four barriers per group; forward and DGrad on 256 x 256 tiles);
//   - LDS rows are 128 bytes with the 16-byte chunks of a row XOR-permuted (see swz) for the fragment reads;
//   - block-scaled B (forward, DGrad): s = fl32(sa * sb) per row and group (the block scale is uniform over
//     the tile); row-scaled B (WGrad): sa * sb per element;
//   - blocks are renumbered so that each XCD (8 per device, dispatched round robin) works on a compact
//     band of output tiles that share A rows and B rows in its L2.
#include "jetfp8_common.h"
#include "jetfp8_launch.h"
#include "jetfp8_mfma.h"

namespace jetfp8 {

constexpr int L_THREADS = 512;
// Block tile of the large-M kernel: 256 x 256 (SPLIT = 1), or 128 x 128 (SPLIT = 2) for the last, partial round
// of tiles and for 65..128-row calls.  8 waves as 2 (rows) x 4 (columns); a wave owns TM x TN 16x16 tiles.  The
// operand tiles are staged in parts of 64 rows (one 1 KB region per wave and part).
template <int SPLIT>
struct LargeCfg {
    static constexpr int BM = 256 / SPLIT, BN = 256 / SPLIT;
    static constexpr int WROWS = BM / 2, WCOLS = BN / 4;          // wave tile
    static constexpr int TM = WROWS / 16, TN = WCOLS / 16;        // 8 x 4 or 4 x 2 tiles of 16x16
    static constexpr int PA = BM / 64, PB = BN / 64;              // staging parts of A and B
    static constexpr int PARTS = PA > PB ? PA : PB;
};

// LDS row layout: 128-byte rows, the 16-byte chunk c of row r stored at chunk c ^ swz(r).  The XOR
// pattern was chosen by measurement on gfx950 (fragment reads at ~170 B/clk/CU against ~113 for the
// plain c ^ (r & 7)); it depends on r & 15 only, so 16-row tiles share one pattern.
__device__ __forceinline__ uint32_t swz(uint32_t r) { return (((r & 7) * 5) & 7) ^ ((r >> 3) & 1); }

#define JETFP8_BUFFER_LOAD_LDS(r, lds, size, voffset, soffset) \
    __builtin_amdgcn_raw_ptr_buffer_load_lds((r), (lds), (size), (voffset), (soffset), 0, 0)

// Work item -> output tile.  Tiles of the 256 x 256 grid (tiles_m x tiles_n) are ordered in bands of `group_m`
// tile-rows, N fastest inside a band; a call covers the band-order range [q_begin, q_begin + q_count).
// SPLIT = 1: the work item is renumbered so that XCD x (which receives blocks x, x+8, ...) owns a contiguous part
// of the range.  Bands of 4 tile-rows measured 1.4 % faster than bands of 8 (fewer L2 misses on the large shapes)
// and bands of 2 or 16 slower.  SPLIT = 2: each 256 x 256 tile is `qrows` x 2 work items, its 128 x 128 quarters
// (qrows = 1: the upper two only), returned in units of the 128 x 128 grid.
template <int SPLIT>
__device__ __forceinline__ void tile_of_work(int w, int tiles_m, int tiles_n, int q_begin, int q_count, int qrows,
                                             int& tm, int& tn) {
    int q, quad = 0;
    if (SPLIT == 1) {
        // (a 256 x 256 call always starts at the first tile: q_begin is 0 and not read, which keeps it out of the
        // scalar registers the kernel's buffer descriptors need)
        const int per = q_count / 8, rem = q_count % 8, xcd = w % 8, idx = w / 8;
        q = xcd * per + (xcd < rem ? xcd : rem) + idx;
    } else {
        q = q_begin + w / (2 * qrows);
        quad = w % (2 * qrows);
    }
    const int group_m = 4;
    const int band = group_m * tiles_n;
    const int first_m = (q / band) * group_m;
    const int gsz = min(tiles_m - first_m, group_m);
    const int wb = q % band;
    tm = first_m + wb % gsz;
    tn = wb / gsz;
    if (SPLIT == 2) {
        tm = 2 * tm + quad / 2;
        tn = 2 * tn + quad % 2;
    }
}

// One ring stage: A tile, B tile and the scales of one group.  Distinct LDS objects (not one array
// indexed by a run-time stage) let the compiler see that the stage being filled by the direct-to-LDS loads
// is not the stage being read, so it does not drain the loads before every LDS read.
template <int SPLIT>
struct __attribute__((aligned(1024))) LargeStage {
    uint8_t a[LargeCfg<SPLIT>::BM * BK];
    uint8_t b[LargeCfg<SPLIT>::BN * BK];
    float sa[LargeCfg<SPLIT>::BM];    // row scales of A
    float sb[LargeCfg<SPLIT>::BN];    // row scales of B (WGrad)
};

// Per-tile values shared by the block: output tile coordinates and the buffer descriptors of the tile's
// operand bands and scale rows.  Built from block-uniform values only, so everything stays in scalar
// registers.
struct TileCtx {
    int tmi, tni;          // tile row / column
    int i0, j0;            // first output row / column
    rsrc_t ra, rb;         // A rows i0 .. i0+BM-1, B rows j0 .. j0+BN-1 (clipped to I, J)
    rsrc_t rsa, rsb;       // A-row scales from i0; B-row scales from j0 (row-scaled B only)
};

template <bool ROW_SCALED_B, int SPLIT>
__global__ __launch_bounds__(L_THREADS, SPLIT) void gemm_large_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, uint16_t* __restrict__ Cout, int64_t I, int64_t J, int64_t Kc, int64_t sbj,
    int64_t sbg, int tiles_m, int tiles_n, int q_begin, int q_count, int qrows) {
    using Cfg = LargeCfg<SPLIT>;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, WROWS = Cfg::WROWS, WCOLS = Cfg::WCOLS, TM = Cfg::TM, TN = Cfg::TN;
    typedef LargeStage<SPLIT> Stage;
    // 2-deep ring: while group g is multiplied, the next group is in flight.
    __shared__ Stage stage0, stage1;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);     // wave-uniform, kept in scalar registers
    const int wm = wave >> 2, wn = wave & 3;                      // wave tile: rows wm*WROWS.., cols wn*WCOLS..
    const int G = (int)(Kc / BK);
    const int T = SPLIT == 1 ? q_count : q_count * 2 * qrows;      // work items (tiles) of this call
    // Persistent blocks: block b computes tiles b, b + gridDim.x, ... one after the other; the ring and its
    // prefetch run on across tile boundaries, and a tile's output is stored while the next tile's first
    // group is multiplied (row of tiles tm just before that row's first promotion).  Every block has at least
    // one tile (grid <= number of tiles).
    // (the division runs on the vector unit; readfirstlane marks the uniform result as scalar, so every condition
    // derived from it stays a scalar branch)
    const int nsteps = __builtin_amdgcn_readfirstlane(((T - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * G);

    auto tile_ctx = [&](int pid) __attribute__((always_inline)) -> TileCtx {
        TileCtx c;
        int tm_, tn_;
        tile_of_work<SPLIT>(pid, tiles_m, tiles_n, q_begin, q_count, qrows, tm_, tn_);
        // the tile index is block-uniform; the integer divisions above run on the vector unit, so say so
        c.tmi = __builtin_amdgcn_readfirstlane(tm_);
        c.tni = __builtin_amdgcn_readfirstlane(tn_);
        c.i0 = c.tmi * BM;
        c.j0 = c.tni * BN;
        // 32-bit scalar arithmetic: all dims are < 2^31 and operand bands < 2^31 bytes.  A 128 x 128 quarter of a
        // 256 x 256 tile can lie wholly past I or J: its descriptors are then empty (loads read zero) and none of
        // its outputs is stored.  The clamps compile to a vector median instruction; readfirstlane returns the
        // (uniform) results to scalar registers, so the descriptors stay scalar (in vector registers every buffer
        // load would be wrapped in a loop over the distinct descriptors of the wave).
        const int rows_a = __builtin_amdgcn_readfirstlane(max(0, min((int)I - c.i0, BM)));
        const int rows_b = __builtin_amdgcn_readfirstlane(max(0, min((int)J - c.j0, BN)));
        const int sa_bytes = __builtin_amdgcn_readfirstlane(max(0, G * (int)I - c.i0) * 4);
        const int sb_bytes = ROW_SCALED_B ? __builtin_amdgcn_readfirstlane(max(0, G * (int)J - c.j0) * 4) : 0;
        c.ra = make_rsrc(A + (int64_t)c.i0 * Kc, rows_a * (int)Kc);
        c.rb = make_rsrc(B + (int64_t)c.j0 * Kc, rows_b * (int)Kc);
        c.rsa = make_rsrc(As + c.i0, sa_bytes);
        c.rsb = make_rsrc(Bs + (ROW_SCALED_B ? c.j0 : 0), sb_bytes);
        return c;
    };

    // ---- global -> LDS staging with buffer loads, spread over the first four row tiles of the previous
    //      group (one A and one B instruction per wave per tile) so that no wave stalls on a burst of load
    //      issues and the fragment reads at the start of a group meet no load traffic.  Each operand has a
    //      scalar descriptor over the tile's row band, so rows past I (or J) read as zero and are never
    //      stored.  Part c of wave w fills the 1 KB LDS region (8 c + w) of A and of B: rows 64 c + 8 w ..
    //      +7; lane l lands at row +l/8, physical chunk l%8.  The row's swizzle depends on r & 15 only, so
    //      one lane offset serves all c, and the c and group terms go into the scalar offset.  Scales (with
    //      part 0): one dword per lane, waves 0..3 bring 64 A-row scales each, waves 4..7 (row-scaled B)
    //      64 B-row scales each; out-of-range rows read as zero.
    const uint32_t r0 = wave * 8 + (lane >> 3);
    const int ooff = (int)(r0 * (uint32_t)Kc + (((lane & 7) ^ swz(r0)) << 4));
    const int cstep = 64 * (int)Kc;
    const int os = ((wave & 3) * 64 + lane) * 4;
    auto issue_part = [&](int c, const TileCtx& tc, int g, Stage& S) __attribute__((always_inline)) {
        if (c == 0) {
            if (wave < Cfg::PA) JETFP8_BUFFER_LOAD_LDS(tc.rsa, (lds_void*)&S.sa[wave * 64], 4, os, g * (int)I * 4);
            else if (ROW_SCALED_B && wave >= 4 && wave - 4 < Cfg::PB)
                JETFP8_BUFFER_LOAD_LDS(tc.rsb, (lds_void*)&S.sb[(wave - 4) * 64], 4, os, g * (int)J * 4);
        }
        const int go = g * BK + c * cstep;
        if (c < Cfg::PA) JETFP8_BUFFER_LOAD_LDS(tc.ra, (lds_void*)(&S.a[(c * 8 + wave) * 1024]), 16, ooff, go);
        if (c < Cfg::PB) JETFP8_BUFFER_LOAD_LDS(tc.rb, (lds_void*)(&S.b[(c * 8 + wave) * 1024]), 16, ooff, go);
    };

    v4f acc[TM][TN];
#pragma unroll
    for (int a = 0; a < TM; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    const int qc4 = 4 * (lane >> 4);       // first of the 4 output columns of this lane inside a 16x16 tile
    // Fragment bytes of this lane: row (lane & 15) of each 16-row tile, logical chunks cp and cp + 1.  The
    // tile's first row is a multiple of 16, so the swizzle depends on (lane & 15) only and consecutive
    // tiles are 2048 bytes apart: one base offset per chunk, tiles by immediate offsets.
    const uint32_t rl = lane & 15, cp = 2 * (lane >> 4), sw = swz(rl);
    const uint32_t fa0 = (wm * WROWS + rl) * BK + ((cp ^ sw) << 4), fa1 = (wm * WROWS + rl) * BK + (((cp + 1) ^ sw) << 4);
    const uint32_t fb0 = (wn * WCOLS + rl) * BK + ((cp ^ sw) << 4), fb1 = (wn * WCOLS + rl) * BK + (((cp + 1) ^ sw) << 4);

    // Output of one row of 16x16 tiles: bf16, round to nearest even; each lane writes 4 consecutive columns
    // (8 bytes) per tile.  J is a multiple of 128, so a lane's 4 columns are either all inside J or all
    // outside.  The accumulators of the row are cleared for the next tile.
    auto store_row = [&](int tm, int i0, int j0) __attribute__((always_inline)) {
        const int64_t r = i0 + wm * WROWS + tm * 16 + rl;
        if (r < I) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int64_t c = j0 + wn * WCOLS + tn * 16 + qc4;
                if (c < J) {
                    uint2 w;
                    w.x = f32_to_bf16_rne(acc[tm][tn][0]) | (f32_to_bf16_rne(acc[tm][tn][1]) << 16);
                    w.y = f32_to_bf16_rne(acc[tm][tn][2]) | (f32_to_bf16_rne(acc[tm][tn][3]) << 16);
                    *reinterpret_cast<uint2*>(&Cout[r * J + c]) = w;
                }
            }
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    };

    // compute cursor (tile, group) and issue cursor (one step ahead)
    int cpid = blockIdx.x, cg = 0;
    TileCtx cur = tile_ctx(cpid);
    int ipid = cpid, ig = 0;
    TileCtx iss = cur;
    int prev_i0 = 0, prev_j0 = 0;
    auto advance_issue = [&]() __attribute__((always_inline)) {
        if (++ig == G) {
            ig = 0;
            ipid += gridDim.x;
            if (ipid < T) iss = tile_ctx(ipid);
        }
    };

    // Block scale of B (forward, DGrad) for the group being multiplied, fetched one step ahead with a
    // vector load (counted with the staging loads, so the post-barrier fragment reads are not held up by
    // a scalar load in flight).
    const rsrc_t rbs = make_rsrc(Bs, ROW_SCALED_B ? 0 : (int)(J / 128) * G * 4);
    auto load_sb = [&](int j0, int g) __attribute__((always_inline)) -> float {
        const int bblk = min((j0 + wn * WCOLS) / 128, (int)(J / 128) - 1);
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, (bblk * (int)sbj + g * (int)sbg) * 4, 0, 0));
    };
    float sbv_cur = 0.0f, sbv_nxt = 0.0f;

    // One step: wait for the current group's stage, store the previous tile at a tile's first group,
    // multiply, and (during the first row tiles) refill the other stage (read one step ago) with the next
    // group, of this tile or of the block's next tile.
    auto step = [&](int s, Stage& S, Stage& refill) __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);   // keep each group's code in place (bounded register pressure)
        // this wave's loads of this group landed, its LDS reads of the previous one returned and its
        // stores of the previous tile completed; then every wave of the block is past that point
        __builtin_amdgcn_s_setprio(0);
        __builtin_amdgcn_s_waitcnt(0);
        __builtin_amdgcn_s_barrier();
        // The refill of the other stage is issued in every step, the last one included: there the issue cursor
        // still points at a valid group (of the block's last tile) and nothing reads that stage any more.  A guard
        // on it cost a vector select and compare per row tile (the compiler negates a uniform branch condition as
        // a lane mask).  Flags below are scalar integers (readfirstlane) for the same reason.
        // first group of a tile after the first: the previous tile's rows are stored one row of tiles at a
        // time, each just before its first promotion, so the stores spread over the group.  Row-scaled B
        // (long contraction, few tiles per block, no register room in the hot loop) stores the whole tile
        // here instead.
        const bool first_of_tile = cg == 0 && s > 0;
        const bool flush = !ROW_SCALED_B && first_of_tile;
        if (ROW_SCALED_B && first_of_tile) {
#pragma unroll
            for (int tm = 0; tm < TM; ++tm) store_row(tm, prev_i0, prev_j0);
        }
        // block-scaled B: one scale per (128-block of B rows, group); a wave's 64 columns lie in one block.
        // Columns past J (last tile when J is an odd multiple of 128) use the last block: never stored.
        const float sbv = sbv_cur;

        // The matrix op takes the B fragment as its first operand, so lane l holds output row (l & 15) of
        // each 16-row tile and the 4 consecutive columns 4 * (l >> 4) .. +3: one A-row scale per tile.
        float s1[TM];
        const float* sar = S.sa + (wm * WROWS + (int)rl);   // tiles by immediate offsets
#pragma unroll
        for (int tm = 0; tm < TM; ++tm) {
            s1[tm] = sar[tm * 16];
            if (!ROW_SCALED_B) s1[tm] = s1[tm] * sbv;            // s = fl32(sa * sb)
        }
        v4f sb4[TN];
        if (ROW_SCALED_B) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) sb4[tn] = *reinterpret_cast<const v4f*>(S.sb + (wn * WCOLS + qc4) + tn * 16);
        }
        v8i bfr[TN];
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) {
            const uint4 lo = *reinterpret_cast<const uint4*>(&S.b[fb0 + tn * 2048]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&S.b[fb1 + tn * 2048]);
            bfr[tn] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        auto a_frag = [&](int tm) __attribute__((always_inline)) -> v8i {
            const uint4 lo = *reinterpret_cast<const uint4*>(&S.a[fa0 + tm * 2048]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&S.a[fa1 + tm * 2048]);
            return (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        };
        auto promote = [&](int tm, const v4f* p) __attribute__((always_inline)) {
            if (flush) store_row(tm, prev_i0, prev_j0);
            // row-scaled B: the tile's 16 scale products are formed here; the pinned copy of the row scale
            // keeps the compiler from forming all 128 of a group at once
            float srow = s1[tm];
            if (ROW_SCALED_B) asm volatile("" : "+v"(srow));
#pragma unroll
            for (int tn = 0; tn < TN; ++tn)
#pragma unroll
                for (int v = 0; v < 4; ++v) {
                    const float sc = ROW_SCALED_B ? srow * sb4[tn][v] : srow;
                    acc[tm][tn][v] = fmaf(p[tn][v], sc, acc[tm][tn][v]);
                }
            // pin the promotion here: without this the compiler sinks it below later matrix ops and keeps
            // every group product alive at once
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) asm volatile("" : "+v"(acc[tm][tn]));
        };
        // software pipeline over the 8 row tiles: the matrix ops of tile tm+1 run while tile tm is promoted.
        // Block-scaled B: one product buffer -- tile (tm-1, tn) is promoted right before (tm, tn) is issued
        // into the same registers (the other wave of the SIMD keeps the matrix unit busy meanwhile).
        // Row-scaled B: two buffers, a whole row of tiles issued before the previous row is promoted.
        if (!ROW_SCALED_B) {
            v4f pp[TN];
            v8i af = a_frag(0);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) pp[tn] = mfma_group(bfr[tn], af);
#pragma unroll
            for (int tm = 1; tm < TM; ++tm) {
                af = a_frag(tm);
                if (tm <= Cfg::PARTS) issue_part(tm - 1, iss, ig, refill);
                if (tm == 1) sbv_nxt = load_sb(iss.j0, ig);
                __builtin_amdgcn_sched_barrier(0);
                // Each SIMD runs one wave of each half (wm = 0, 1).  Issue arbitration favours the older wave
                // (wm = 0), which then reaches the step's barrier well before its partner and leaves the matrix
                // unit to a single wave; raising the younger wave's priority for the first half of the step
                // evens out their progress.
                if (wm == 1 && tm < TM / 2) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                if (flush) store_row(tm - 1, prev_i0, prev_j0);
#pragma unroll
                for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
                    for (int v = 0; v < 4; ++v) acc[tm - 1][tn][v] = fmaf(pp[tn][v], s1[tm - 1], acc[tm - 1][tn][v]);
                    asm volatile("" : "+v"(acc[tm - 1][tn]));
                    pp[tn] = mfma_group(bfr[tn], af);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            if (flush) store_row(TM - 1, prev_i0, prev_j0);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[TM - 1][tn][v] = fmaf(pp[tn][v], s1[TM - 1], acc[TM - 1][tn][v]);
                asm volatile("" : "+v"(acc[TM - 1][tn]));
            }
            __builtin_amdgcn_sched_barrier(0);
        } else {
            v4f pa[TN], pb[TN];
            v8i af = a_frag(0);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) pa[tn] = mfma_group(bfr[tn], af);
#pragma unroll
            for (int tm = 1; tm < TM; ++tm) {
                af = a_frag(tm);
                if (tm <= Cfg::PARTS) issue_part(tm - 1, iss, ig, refill);
                __builtin_amdgcn_sched_barrier(0);
                if (wm == 1 && tm < TM / 2) __builtin_amdgcn_s_setprio(1);
                else __builtin_amdgcn_s_setprio(0);
                if (tm & 1) {
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) pb[tn] = mfma_group(bfr[tn], af);
                    promote(tm - 1, pa);
                } else {
#pragma unroll
                    for (int tn = 0; tn < TN; ++tn) pa[tn] = mfma_group(bfr[tn], af);
                    promote(tm - 1, pb);
                }
            }
            __builtin_amdgcn_sched_barrier(0);
            promote(TM - 1, pb);
            __builtin_amdgcn_sched_barrier(0);
        }
        advance_issue();
        if (!ROW_SCALED_B) sbv_cur = sbv_nxt;
        // advance the compute cursor
        if (++cg == G) {
            cg = 0;
            prev_i0 = cur.i0;
            prev_j0 = cur.j0;
            cpid += gridDim.x;
            if (cpid < T) cur = tile_ctx(cpid);
        }
    };

#pragma unroll
    for (int c = 0; c < Cfg::PARTS; ++c) issue_part(c, iss, ig, stage0);
    if (!ROW_SCALED_B) sbv_cur = load_sb(iss.j0, ig);
    advance_issue();
    int s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        step(s, stage0, stage1);
        step(s + 1, stage1, stage0);
    }
    if (s < nsteps) step(s, stage0, stage1);
    // the last step's refill loads are still in flight: they must land before the block's LDS is released
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int tm = 0; tm < TM; ++tm) store_row(tm, prev_i0, prev_j0);
}

// ---- forward / DGrad on 256 x 256 tiles: the two waves of each SIMD in alternating phases --------------------
// The same tiles, staging ring, LDS layout and per-element operation sequence as gemm_large_kernel (so the same
// bits), scheduled so that the matrix unit of a SIMD is fed by one wave at a time while its partner reads LDS:
//   - a group is two halves (row tiles 0-3, 4-7 of the wave tile); each half is a memory phase (the half's A
//     fragments and row scales, at the first half also the B fragments, then staging loads for the ring) and a
//     compute phase (16 matrix ops, each preceded in issue order by the promotion of the previous row tile's
//     product of the same column tile, so the VALU works under the matrix unit);
//   - waves 0-3 (wm = 0, one per SIMD) run one phase ahead of waves 4-7 (wm = 1): between two block barriers
//     one wave of each SIMD computes while the other loads.  Register-only measurement on gfx950: one wave issuing
//     matrix op + 4 promotion FMAs in this order keeps the matrix unit 90 % as busy as matrix ops alone; 16 FMAs
//     followed by 4 matrix ops (the order the compiler picks for the interleaved-waves kernel) only 61 %;
//   - the promotion lags one row tile, across phases too: row tile 7 of a group is promoted at the start of the
//     next group's first compute phase.  Rows 0-2 of a tile are final after the first compute phase of its last
//     group and are stored in the next memory phase; rows 3-6 and row 7 in the memory phases of the next tile's
//     first group;
//   - the refill of the ring is spread over all four memory phases of a group (see the staging comment below);
//   - a wave raises its issue priority in its memory phases, so its reads and loads are not held up behind the
//     partner's matrix ops.
__global__ __launch_bounds__(L_THREADS, 1) void gemm_pp_kernel(
    const uint8_t* __restrict__ A, const float* __restrict__ As, const uint8_t* __restrict__ B,
    const float* __restrict__ Bs, uint16_t* __restrict__ Cout, int64_t I, int64_t J, int64_t Kc, int64_t sbj,
    int64_t sbg, int tiles_m, int tiles_n, int q_count) {
    using Cfg = LargeCfg<1>;
    constexpr int BM = Cfg::BM, BN = Cfg::BN, WROWS = Cfg::WROWS, WCOLS = Cfg::WCOLS, TN = Cfg::TN;
    typedef LargeStage<1> Stage;
    __shared__ Stage stage0, stage1;

    const int t = threadIdx.x, lane = t & 63;
    const int wave = __builtin_amdgcn_readfirstlane(t >> 6);
    const int wm = wave >> 2, wn = wave & 3;
    const int G = (int)(Kc / BK);
    const int T = q_count;
    const int nsteps = __builtin_amdgcn_readfirstlane(((T - 1 - (int)blockIdx.x) / (int)gridDim.x + 1) * G);

    auto tile_ctx = [&](int pid) __attribute__((always_inline)) -> TileCtx {
        TileCtx c;
        int tm_, tn_;
        tile_of_work<1>(pid, tiles_m, tiles_n, 0, q_count, 1, tm_, tn_);
        c.tmi = __builtin_amdgcn_readfirstlane(tm_);
        c.tni = __builtin_amdgcn_readfirstlane(tn_);
        c.i0 = c.tmi * BM;
        c.j0 = c.tni * BN;
        const int rows_a = __builtin_amdgcn_readfirstlane(min((int)I - c.i0, BM));
        const int rows_b = __builtin_amdgcn_readfirstlane(min((int)J - c.j0, BN));
        const int sa_bytes = __builtin_amdgcn_readfirstlane((G * (int)I - c.i0) * 4);
        c.ra = make_rsrc(A + (int64_t)c.i0 * Kc, rows_a * (int)Kc);
        c.rb = make_rsrc(B + (int64_t)c.j0 * Kc, rows_b * (int)Kc);
        c.rsa = make_rsrc(As + c.i0, sa_bytes);
        c.rsb = c.rsa;                                           // unused here: B is block-scaled
        return c;
    };

    // staging: the LDS layout of gemm_large_kernel (1 KB region q of an operand tile holds rows 8 q .. 8 q + 7; lane
    // l lands at row + l / 8, physical chunk l % 8).  Part c = rows 64 c .. 64 c + 63 of A or B: one wave issues two
    // regions of it, 8 c + (w & 3) and 8 c + (w & 3) + 4, so the 4 waves of one phase cover a part.
    //   - A parts of the next group: waves 0-3 parts 0 and 2 in their first memory phase, waves 4-7 parts 1 and 3
    //     in theirs (one phase later); with them the A-row scales of those parts (waves 0, 1, 4, 5);
    //   - B parts of the group after next (the B tile of the current stage is read by then): waves 0-3 parts 0
    //     and 1, waves 4-7 parts 2 and 3, in their second memory phases.
    // Each wave then issues 4 staging loads per memory phase; all of them in one phase made that phase the
    // critical path (the issue of direct-to-LDS loads stalls the wave).  A wave waits for its loads at the end of
    // its next second memory phase; the first read of each part comes at least one phase later.
    const uint32_t rq = (wave & 3) * 8 + (lane >> 3);
    const int qoff = (int)(rq * (uint32_t)Kc + (((lane & 7) ^ swz(rq)) << 4));   // rows +32: same swizzle
    const int cstep = 64 * (int)Kc;
    auto issue_rows = [&](rsrc_t r, uint8_t* base, int c, int g) __attribute__((always_inline)) {
        const int go = g * BK + c * cstep;
        JETFP8_BUFFER_LOAD_LDS(r, (lds_void*)(base + (c * 8 + (wave & 3)) * 1024), 16, qoff, go);
        JETFP8_BUFFER_LOAD_LDS(r, (lds_void*)(base + (c * 8 + (wave & 3) + 4) * 1024), 16, qoff, go + 32 * (int)Kc);
    };
    auto issue_a = [&](const TileCtx& tc, int g, Stage& S) __attribute__((always_inline)) {
        issue_rows(tc.ra, S.a, wm, g);
        issue_rows(tc.ra, S.a, wm + 2, g);
        if ((wave & 3) < 2) {
            const int c = wm + 2 * (wave & 1);
            JETFP8_BUFFER_LOAD_LDS(tc.rsa, (lds_void*)&S.sa[c * 64], 4, (c * 64 + lane) * 4, g * (int)I * 4);
        }
    };
    auto issue_b = [&](rsrc_t rb, int g, Stage& S) __attribute__((always_inline)) {
        issue_rows(rb, S.b, 2 * wm, g);
        issue_rows(rb, S.b, 2 * wm + 1, g);
    };

    v4f acc[8][TN];
#pragma unroll
    for (int a = 0; a < 8; ++a)
#pragma unroll
        for (int b = 0; b < TN; ++b) acc[a][b] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};

    const int qc4 = 4 * (lane >> 4);
    const uint32_t rl = lane & 15, cp = 2 * (lane >> 4), sw = swz(rl);
    const uint32_t fa0 = (wm * WROWS + rl) * BK + ((cp ^ sw) << 4), fa1 = (wm * WROWS + rl) * BK + (((cp + 1) ^ sw) << 4);
    const uint32_t fb0 = (wn * WCOLS + rl) * BK + ((cp ^ sw) << 4), fb1 = (wn * WCOLS + rl) * BK + (((cp + 1) ^ sw) << 4);

    auto store_row = [&](int tm, int i0, int j0) __attribute__((always_inline)) {
        const int64_t r = i0 + wm * WROWS + tm * 16 + rl;
        if (r < I) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const int64_t c = j0 + wn * WCOLS + tn * 16 + qc4;
                if (c < J) {
                    uint2 w;
                    w.x = f32_to_bf16_rne(acc[tm][tn][0]) | (f32_to_bf16_rne(acc[tm][tn][1]) << 16);
                    w.y = f32_to_bf16_rne(acc[tm][tn][2]) | (f32_to_bf16_rne(acc[tm][tn][3]) << 16);
                    *reinterpret_cast<uint2*>(&Cout[r * J + c]) = w;
                }
            }
        }
#pragma unroll
        for (int tn = 0; tn < TN; ++tn) acc[tm][tn] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    };

    int cpid = blockIdx.x, cg = 0;
    TileCtx cur = tile_ctx(cpid);
    // issue cursors: A (and the block scale) one group ahead of the compute cursor, B two groups ahead.  Past the
    // block's last group a cursor stays on a valid group of the last tile (loaded, never read).
    int ipid = cpid, ig = 0;
    TileCtx iss = cur;
    int bpid = cpid, bg = 0;
    rsrc_t rbb = cur.rb;
    int prev_i0 = 0, prev_j0 = 0;
    auto advance_issue = [&]() __attribute__((always_inline)) {
        if (++ig == G) {
            ig = 0;
            ipid += gridDim.x;
            if (ipid < T) iss = tile_ctx(ipid);
        }
    };
    auto advance_b = [&]() __attribute__((always_inline)) {
        if (++bg == G) {
            bg = 0;
            bpid += gridDim.x;
            if (bpid < T) rbb = tile_ctx(bpid).rb;
        }
    };
    const rsrc_t rbs = make_rsrc(Bs, (int)(J / 128) * G * 4);
    auto load_sb = [&](int j0, int g) __attribute__((always_inline)) -> float {
        const int bblk = min((j0 + wn * WCOLS) / 128, (int)(J / 128) - 1);
        return __uint_as_float(__builtin_amdgcn_raw_buffer_load_b32(rbs, (bblk * (int)sbj + g * (int)sbg) * 4, 0, 0));
    };
    float sbv_cur = 0.0f, sbv_nxt = 0.0f;

    // block barrier between phases; the empty asm with a memory clobber keeps every LDS access on its side
    auto sync = [&]() __attribute__((always_inline)) {
        __builtin_amdgcn_sched_barrier(0);
        __builtin_amdgcn_s_barrier();
        asm volatile("" ::: "memory");
        __builtin_amdgcn_sched_barrier(0);
    };

    v8i bfr[TN], afr[4];
    v4f pp[TN];
#pragma unroll
    for (int tn = 0; tn < TN; ++tn) pp[tn] = (v4f){0.0f, 0.0f, 0.0f, 0.0f};
    float s1[4];
    float s_prev = 0.0f;   // scale of the row tile whose products are in pp (the first promotion adds +0 to +0)

    // memory phase: the half's A fragments (and at the first half the B fragments) and row scales
    auto read_half = [&](const Stage& S, int hf) __attribute__((always_inline)) {
        if (hf == 0) {
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
                const uint4 lo = *reinterpret_cast<const uint4*>(&S.b[fb0 + tn * 2048]);
                const uint4 hi = *reinterpret_cast<const uint4*>(&S.b[fb1 + tn * 2048]);
                bfr[tn] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
            }
        }
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int tm = 4 * hf + i;
            const uint4 lo = *reinterpret_cast<const uint4*>(&S.a[fa0 + tm * 2048]);
            const uint4 hi = *reinterpret_cast<const uint4*>(&S.a[fa1 + tm * 2048]);
            afr[i] = (v8i){(int)lo.x, (int)lo.y, (int)lo.z, (int)lo.w, (int)hi.x, (int)hi.y, (int)hi.z, (int)hi.w};
        }
        const float* sar = S.sa + (wm * WROWS + (int)rl);
#pragma unroll
        for (int i = 0; i < 4; ++i) s1[i] = sar[(4 * hf + i) * 16] * sbv_cur;     // s = fl32(sa * sb)
    };

    // compute phase: row tiles 4 hf .. 4 hf + 3.  Before the matrix op (r, tn) the product of (r - 1, tn) (row 7 of
    // the previous group for r = 0) is promoted out of the same registers; the empty asm statements fix this order.
    // Issue priority: 1 in the memory phases, 0 in the compute phases, so that the reading wave's LDS and load
    // instructions are not held up behind its partner's matrix ops (measured +2-4 % on forward / DGrad against
    // raising the computing wave instead, and about the same for priority 3 or a raise in the first memory phase
    // only).
    auto compute_half = [&](int hf) __attribute__((always_inline)) {
        __builtin_amdgcn_s_setprio(0);
#pragma unroll
        for (int i = 0; i < 4; ++i) {
            const int prev = i > 0 ? 4 * hf + i - 1 : (hf == 0 ? 7 : 3);
#pragma unroll
            for (int tn = 0; tn < TN; ++tn) {
#pragma unroll
                for (int v = 0; v < 4; ++v) acc[prev][tn][v] = fmaf(pp[tn][v], s_prev, acc[prev][tn][v]);
                asm volatile("" : "+v"(acc[prev][tn]));
                asm volatile("" : "+v"(bfr[tn]));
                pp[tn] = mfma_group(bfr[tn], afr[i]);
                asm volatile("" : "+v"(pp[tn]));
            }
            s_prev = s1[i];
        }
    };

    auto group = [&](int s, Stage& S, Stage& R) __attribute__((always_inline)) {
        const bool first_of_tile = cg == 0 && s > 0;
        __builtin_amdgcn_s_setprio(1);
        // ---- memory phase, first half
        if (first_of_tile) {
#pragma unroll
            for (int tm = 3; tm < 7; ++tm) store_row(tm, prev_i0, prev_j0);
        }
        // fragment reads first, then the staging loads (loads first measured 2.5-4 % slower on forward / DGrad;
        // waiting for the reads before issuing the loads, 1-3 % slower)
        read_half(S, 0);
        __builtin_amdgcn_sched_barrier(0);
        issue_a(iss, ig, R);
        sbv_nxt = load_sb(iss.j0, ig);
        __builtin_amdgcn_s_waitcnt(kWaitLgkm0);
        sync();
        compute_half(0);
        sync();
        __builtin_amdgcn_s_setprio(1);
        // ---- memory phase, second half
        if (first_of_tile) store_row(7, prev_i0, prev_j0);
        if (cg == G - 1) {
#pragma unroll
            for (int tm = 0; tm < 3; ++tm) store_row(tm, cur.i0, cur.j0);
        }
        read_half(S, 1);
        // this wave's staging loads of the previous memory phases have landed, and its fragment reads have returned
        __builtin_amdgcn_s_waitcnt(0);
        issue_b(rbb, bg, S);
        sync();
        compute_half(1);
        sync();
        advance_issue();
        advance_b();
        sbv_cur = sbv_nxt;
        if (++cg == G) {
            cg = 0;
            prev_i0 = cur.i0;
            prev_j0 = cur.j0;
            cpid += gridDim.x;
            if (cpid < T) cur = tile_ctx(cpid);
        }
    };

    // prologue: the first group whole, and the B tile of the second
    issue_a(iss, ig, stage0);
    issue_b(rbb, bg, stage0);
    sbv_cur = load_sb(iss.j0, ig);
    advance_issue();
    advance_b();
    issue_b(rbb, bg, stage1);
    advance_b();
    __builtin_amdgcn_s_waitcnt(0);
    sync();
    if (wm == 1) sync();     // waves 4-7 run one phase behind waves 0-3
    int s = 0;
    for (; s + 2 <= nsteps; s += 2) {
        group(s, stage0, stage1);
        group(s + 1, stage1, stage0);
    }
    if (s < nsteps) group(s, stage0, stage1);
    if (wm == 0) sync();     // matching barrier count
    // last promotion (row tile 7 of the block's last group), then rows 3-7 of the last tile
#pragma unroll
    for (int tn = 0; tn < TN; ++tn)
#pragma unroll
        for (int v = 0; v < 4; ++v) acc[7][tn][v] = fmaf(pp[tn][v], s_prev, acc[7][tn][v]);
    __builtin_amdgcn_s_waitcnt(0);
#pragma unroll
    for (int tm = 3; tm < 8; ++tm) store_row(tm, prev_i0, prev_j0);
}

template <bool ROW_SCALED_B, int SPLIT>
static hipError_t launch_large_part(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, uint16_t* C,
                                    int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg, int tiles_m,
                                    int tiles_n, int q_begin, int q_count, int qrows, int max_blocks, hipStream_t st) {
    const int items = q_count * (SPLIT == 1 ? 1 : 2 * qrows);
    const int grid = min(items, max_blocks);
    if (!ROW_SCALED_B && SPLIT == 1) {
        hipLaunchKernelGGL(gemm_pp_kernel, dim3(grid), dim3(L_THREADS), 0, st, A, As, B, Bs, C, I, J, Kc, sbj, sbg,
                           tiles_m, tiles_n, q_count);
        return hipGetLastError();
    }
    hipLaunchKernelGGL((gemm_large_kernel<ROW_SCALED_B, SPLIT>), dim3(grid), dim3(L_THREADS), 0, st, A, As, B, Bs, C,
                       I, J, Kc, sbj, sbg, tiles_m, tiles_n, q_begin, q_count, qrows);
    return hipGetLastError();
}

// Large-M schedule.  T tiles of 256 x 256 run on one persistent block per CU (ceil(T / CUs) rounds).  When T is
// at most half the CU count, the whole call runs on 128 x 128 quarter tiles instead (two blocks per CU; for at
// most 128 rows only the upper quarters), so that more CUs share the work.  When the last round is at most half
// full, that round's R tiles run as 4R quarter tiles after the full rounds, at up to two blocks per CU.  Every
// output element goes through the same operation sequence in every variant, so the bits do not change.
template <bool ROW_SCALED_B>
static hipError_t launch_large(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs, uint16_t* C,
                               int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg, hipStream_t st) {
    const int tiles_m = (int)((I + 255) / 256), tiles_n = (int)((J + 255) / 256);
    const int T = tiles_m * tiles_n;
    const int cus = device_cu_count();
    if (2 * T <= cus)
        return launch_large_part<ROW_SCALED_B, 2>(A, As, B, Bs, C, I, J, Kc, sbj, sbg, tiles_m, tiles_n, 0, T,
                                                  I <= 128 ? 1 : 2, 2 * cus, st);
    const int R = T % cus;
    if (T > cus && R > 0 && 2 * R <= cus) {
        hipError_t e = launch_large_part<ROW_SCALED_B, 1>(A, As, B, Bs, C, I, J, Kc, sbj, sbg, tiles_m, tiles_n, 0,
                                                          T - R, 1, cus, st);
        if (e != hipSuccess) return e;
        return launch_large_part<ROW_SCALED_B, 2>(A, As, B, Bs, C, I, J, Kc, sbj, sbg, tiles_m, tiles_n, T - R, R, 2,
                                                  2 * cus, st);
    }
    return launch_large_part<ROW_SCALED_B, 1>(A, As, B, Bs, C, I, J, Kc, sbj, sbg, tiles_m, tiles_n, 0, T, 1, cus, st);
}

hipError_t launch_gemm_block_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                      uint16_t* C, int64_t I, int64_t J, int64_t Kc, int64_t sbj, int64_t sbg,
                                      hipStream_t st) {
    // decode sizes: the small-M schedule (same per-element sequence, so the same bits)
    if (decode_rows_fit(I, Kc)) return launch_decode_rows(A, As, B, Bs, C, I, 0, I, J, Kc, sbj, sbg, st);
    // 65..128 rows with fewer output columns than contraction: the small-M kernel on the first 64 rows, then on
    // the rest (the weights are read twice, but the 16-column slices keep every CU busy where the quarter tiles of
    // the large kernel would number J / 128 only; measured down projection 14336 -> 4096 at 128 rows: 98 us
    // against 125 us on quarter tiles).  Wider outputs use the quarter tiles (gate_up 4096 -> 28672: 46 us
    // against 168 us).
    if (I <= 128 && J < Kc && decode_rows_fit(64, Kc)) {
        const hipError_t e = launch_decode_rows(A, As, B, Bs, C, I, 0, 64, J, Kc, sbj, sbg, st);
        if (e != hipSuccess) return e;
        return launch_decode_rows(A, As, B, Bs, C, I, 64, I - 64, J, Kc, sbj, sbg, st);
    }
    return launch_large<false>(A, As, B, Bs, C, I, J, Kc, sbj, sbg, st);
}

hipError_t launch_gemm_row_scaled_b(const uint8_t* A, const float* As, const uint8_t* B, const float* Bs,
                                    uint16_t* C, int64_t I, int64_t J, int64_t Kc, hipStream_t st) {
    return launch_large<true>(A, As, B, Bs, C, I, J, Kc, 0, 0, st);
}

}  // namespace jetfp8
