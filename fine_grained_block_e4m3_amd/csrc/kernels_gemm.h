// kernels_gemm.h -- block-scaled E4M3 NT GEMM for gfx950 (MI355X, CDNA4)
// through the FP8 matrix instruction: the opt-in FP8_FLAG_FAST_ACCUM path of
// the block-scaled calls, and the MXFP8 / MXFP4-weight calls.  (The default
// block-scaled path, with exact block partials, is kernels_exact.h.)
//
// Computes Y = X * W^T (BF16 out) with X (M,K) E4M3 + one FP32 scale per 1x128
// tile of a row, W (N,K) E4M3 + one FP32 scale per 128x128 block.
//   Y[m][n] = sum_kb sa[kb][m] * sb[n/128][kb] * P_kb[m][n],
//   P_kb[m][n] = sum_{k in block kb} X[m][k] * W[n][k]
// (tcgen05 page, section 6.1: block-scaled GEMM definition; mlc.ai page,
// "Block-Scaled MMA": output (m,n) uses the scale of row m of A and of row n
// of B; DeepGEMM page, section "主循环骨架": the FP32 partial of each 128-K
// block is multiplied by sA*sB and added to a full-precision accumulator).
//
// gfx950 mapping
//   * One v_mfma_f32_16x16x128_f8f6f4 covers exactly one 128-K block of a
//     16x16 output subtile, so every block partial P_kb is one instruction
//     with a zero accumulator; the promotion acc += (sA*sB)*P_kb is four
//     VALU FMAs in VGPRs that run beside the matrix core.
//   * The W fragment is the MFMA "A" operand and the X fragment the "B"
//     operand.  In the 16x16 f32 result, lane l holds rows 4*(l/16)+r (r=0..3)
//     of column l%16, so a lane owns one m and four consecutive n: one sA
//     value per subtile, and a 16-wide subtile always lies inside one
//     128-row block of W, so sB is uniform over the wave per subtile.
//   * Per K block a wave keeps the fragments of one operand resident in
//     registers and streams the other through, one 16-row subtile at a time:
//     X streams for most instances, W for the 256x224 one (it has more W
//     subtiles per wave than X subtiles).
//   * FP8_FLAG_UE8M0 (power-of-two scales): the scales are fed to
//     v_mfma_scale_f32_16x16x128_f8f6f4 as E8M0 operands and the whole K
//     loop accumulates inside the matrix core -- no VALU promotion.
//   * Operands reach LDS with buffer_load_dwordx4 ... lds (no VGPR staging)
//     through per-tile buffer resources whose range ends at the last valid
//     row: rows past it (M edge, masked rows past the count, N edge) are
//     fetched as zeros by the hardware range check, never from memory.
//     Each tile row is one 128-byte K block; its eight 16-byte chunks are
//     XOR-swizzled by the row index so the fragment reads (16 rows, same
//     chunk) hit distinct banks.  The activation scales of the tile's rows
//     ride in the same stage (one direct-to-LDS dword load per wave).  A ring
//     of STAGES buffers keeps STAGES-1 K blocks in flight; each wave waits on
//     its own vector-memory counter for the oldest stage, then one workgroup
//     barrier publishes it.
//   * Per 128-K block the wave issues the MFMAs of subtile column j while the
//     VALU promotes the partials of column j-1, so matrix core and VALU work
//     side by side (DeepGEMM page, "主循环骨架": promotion on the CUDA cores
//     overlaps the tensor-core work).
//   * Precision.  The FP8 instruction does not sum the 128 products of a block
//     exactly: within each group of 8 consecutive K it truncates every product
//     to a multiple of 2^(E-13), 2^E the group's largest product (measured on
//     gfx950, the analog of the limited FP8 accumulation the DeepGEMM page,
//     section "细粒度缩放在 GEMM 层面引爆的两个问题", reports for H800).
//   * Other paths of the same kernel (template PATH): MXFP8 with 1x32 E8M0
//     scales on both operands and MXFP4 (E2M1) weights; QOUT writes the
//     output as E4M3 with 1x128 scales instead of BF16.  Decode-sized GEMMs with M <= 32 run a kernel of their
//     own (kernels_decode.h).
//   * Persistent grid: each workgroup walks tiles with stride gridDim.x
//     (DeepGEMM page, "线程组织": persistent launch with an in-kernel block
//     scheduler; "统一块调度器与 rasterization": grouped raster order so tiles
//     running together share operand rows in L2).
#pragma once

#include "gemm_common.h"

namespace fp8k {


// How each 128-K block partial is formed.
//   kPathFp8       one FP8 MFMA (16x16x128) per block, VALU promotion by sA*sB
//   kPathFp8Pow2   power-of-two scales as E8M0 operands of the scaled FP8 MFMA,
//                  accumulated over all of K inside the matrix core
//   kPathMx        MXFP8: one E8M0 byte per 1x32 group on both operands (tcgen05
//                  page, sections 6.1 and 6.3: SV = 32, E8M0 scales), packed
//                  4 to a dword per (K block, row) in [K/128][rows] tables.
//                  Each lane passes the byte of the 32-group it holds as its
//                  scale operand and the matrix core accumulates over all of K.
//   kPathMxW4      as kPathMx with W in MXFP4: E2M1 nibbles, two per byte along
//                  K (tcgen05 page, sections 6.3 and the operand-major notes),
//                  64 bytes per row and K block; the instruction's A operand
//                  in E2M1 format.
enum GemmPath : int { kPathFp8 = 0, kPathFp8Pow2 = 1, kPathMx = 2, kPathMxW4 = 3 };

// A 16x128 E4M3 fragment of a lane from LDS: 16 bytes at base+a0 and 16 at
// base+a1, as four 8-byte reads.
__device__ __forceinline__ i32x8 lds_frag(const uint8_t* base, uint32_t a0, uint32_t a1) {
    const i32x2 p = *reinterpret_cast<const i32x2*>(base + a0);
    const i32x2 q = *reinterpret_cast<const i32x2*>(base + a0 + 8);
    const i32x2 r = *reinterpret_cast<const i32x2*>(base + a1);
    const i32x2 t = *reinterpret_cast<const i32x2*>(base + a1 + 8);
    return i32x8{p[0], p[1], q[0], q[1], r[0], r[1], t[0], t[1]};
}

// QOUT: the epilogue emits the output quantized for the next GEMM -- E4M3
// codes and one FP32 scale per 1x128 group along N, [N/128][M] -- instead of
// BF16 (DeepGEMM page, section "为什么只做 NT 布局": the activation
// quantization belongs fused into the kernel that produces the activations).
template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE, int PATH, int STAGES, bool QOUT = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_kernel(
    const uint8_t* __restrict__ xq_, const float* __restrict__ sa_, const uint8_t* __restrict__ wq_,
    const float* __restrict__ sb_, uint16_t* __restrict__ y_, const int32_t* __restrict__ m_indices_,
    const int32_t* __restrict__ masked_m_, GemmParams p) {
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int TM = BM / WAVES_M;   // wave tile rows (m)
    constexpr int TN = BN / WAVES_N;   // wave tile columns (n)
    constexpr int FI = TM / 16;        // 16x16 subtiles per wave along m
    constexpr int FJ = TN / 16;        // ... along n
    // W with E2M1 elements: 64 bytes per row and K block instead of 128
    constexpr bool kW4 = PATH == kPathMxW4;
    constexpr int WROW = kW4 ? 64 : 128;
    constexpr int XLOADS = BM / 8 / NWAVES;   // 1 KB direct-to-LDS loads per wave per stage
    // W rows come in 8-row groups; when they do not split evenly over the
    // waves, the last waves' loads fall past the tile (the range check reads
    // zeros) and land in a spare LDS area, so every wave issues as many.
    constexpr int WGROUPS = BN * WROW / 1024;
    constexpr int WLOADS = (WGROUPS + NWAVES - 1) / NWAVES;
    constexpr int W_WAVES = WGROUPS / WLOADS;   // waves loading rows of the tile
    constexpr int NPIECE = XLOADS + WLOADS + 1;   // loads per wave per stage
    constexpr int PER_STAGE = NPIECE;
    // Scales of a stage: waves 0 .. NSA-1 load the activation scales of the
    // tile's rows (64 each), the other waves each load a copy of the weight
    // scales of the tile's 128-row weight blocks (one per lane).  Every wave
    // issues the same number of loads, so one vmcnt target serves all.
    constexpr int NSA = BM / 64;
    // LDS layout, by operand then stage: [X0 X1 ..][W0 W1 ..][scales0 ..].
    // The operand base lives in the per-lane address and the stage offset in
    // the ds_read immediate.
    constexpr int W_BASE = STAGES * BM * 128;
    constexpr int SC_BASE = W_BASE + STAGES * BN * WROW;
    constexpr int SPARE_BASE = SC_BASE + STAGES * NWAVES * 256;
    // QOUT: the row maxima of each wave column, [WAVES_N][BM] floats
    constexpr int QA_BASE = SPARE_BASE + (W_WAVES < NWAVES ? WLOADS * 1024 : 0);
    constexpr int LDS_BYTES = QA_BASE + (QOUT ? WAVES_N * BM * 4 : 0);
    // A wave's 16-wide n subtiles all lie in one 128-row weight block when its
    // n range is 128-aligned inside a 128-aligned tile: one sB per K block.
    constexpr bool kUniformSb = (BN % 128 == 0 || 128 % BN == 0) && (128 % TN == 0 || TN % 128 == 0)
                                && TN <= 128;
    // Stream the W subtiles (hold X) when a wave has more of them: the
    // resident operand's fragments stay in registers for a whole K block.
    constexpr bool kStreamW = FJ > FI && TM >= 64;
    // With W streamed and FP32 scales, a wave's TN <= 128 columns lie in at
    // most two weight blocks: the K loop is specialised on the subtile where
    // the second one starts, so that the promotion scales are two products
    // per resident fragment and block instead of one per subtile.
    constexpr bool kMx = PATH == kPathMx || PATH == kPathMxW4;
    // scales as E8M0 operands of the scaled MFMA; K accumulated in the matrix core
    constexpr bool kScaledMfma = PATH == kPathFp8Pow2 || kMx;
    // a scale as carried through the pipeline: the FP32 value, or (MX) the
    // E8M0 byte of this lane's 32-group
    using ScaleT = std::conditional_t<kMx, int, float>;
    constexpr bool kSplitSb = kStreamW && TN <= 128 && !kScaledMfma;
    constexpr bool kPow2 = PATH == kPathFp8Pow2;
    static_assert(MODE != kMasked || (!kStreamW && !kSplitSb), "masked: X rows streamed (the skip is per X subtile)");
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole 16x16 subtiles");
    static_assert(BM % 64 == 0 && NSA < NWAVES, "activation scales: 64 rows per wave, one wave left for sB");
    static_assert(BN / 128 + 2 <= 64, "one scale load covers the tile's weight blocks");
    static_assert(BM % (8 * NWAVES) == 0 && (BN * WROW) % 1024 == 0 && WGROUPS % WLOADS == 0,
                  "tile rows per wave");
    static_assert(XLOADS >= 1 && XLOADS <= 4 && WLOADS >= 1 && WLOADS <= 4, "loads per wave");
    static_assert(STAGES >= 2 && LDS_BYTES <= 160 * 1024, "LDS holds the stage ring");
    static_assert((STAGES - 2) * PER_STAGE <= 63, "vmcnt range");
    // MX scales: one dword (a row's 4 bytes of one K block) per tile row and
    // per tile column, one 64-lane dword load per 64 of them
    constexpr int MX_XS_WAVES = BM / 64, MX_WS_WAVES = (BN + 63) / 64;
    static_assert(!kMx || (MODE == kDense && MX_XS_WAVES + MX_WS_WAVES <= NWAVES),
                  "MX: dense only, one scale load per wave");
    static_assert(!QOUT || (MODE == kDense && !kMx && TN == 64 && BN % 128 == 0),
                  "quantized output: dense, 128-column groups of two 64-column waves");

    // A ring of STAGES LDS buffers: the loads of K blocks kb+1 .. kb+STAGES-1
    // fly while block kb is used.
    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    // Masked layout: wave w takes row w / WAVES_N and column w % WAVES_N, so
    // that with WAVES_N = 4 the two waves sharing a SIMD (w mod 4) own
    // different rows (the waves skip the subtiles past an expert's count).
    const int wm = MODE == kMasked ? wave / WAVES_N : wave % WAVES_M;
    const int wn = MODE == kMasked ? wave % WAVES_N : wave / WAVES_M;
    const int64_t K = p.K;
    const int KB = (int)(K / 128);
    const int64_t N = p.N;
    const int g = lane >> 4;             // K group of this lane: bytes [32g, 32g+32)

    int total_tiles = count_tiles<MODE, BM>(p, masked_m_);
    // Contiguous layout on the pair schedule: wave 0 builds it in LDS before
    // the first tile (the planner keeps the blocks within its capacity).
    __shared__ int32_t pair_ent[MODE == kContiguous ? kPairEntries : 1];
    PairShare pair_sh{};
    if constexpr (MODE == kContiguous) {
        if (p.pair_cus > 0) {
            if ((p.M + 127) / 128 > kPairMaxBlocks || p.E > kPairMaxExperts) return;
            if (wave == 0) build_pair_sched(p, m_indices_, pair_ent);
            __syncthreads();
            pair_sh = pair_share<BM, BN>(p, pair_ent);
            total_tiles = pair_sh.units * p.n_tiles;
        }
    }

    // ---- per-lane constants, shared by every tile ----
    // DMA: a wave load fills 1 KB = 8 rows R0..R0+7 of 8-row group grp = R0/8;
    // lane l writes slot l%8 of row R0 + l/8, which must hold logical chunk
    // slot ^ swz(row) = slot ^ (l/8) ^ (grp mod 2).  Source offset within the
    // tile: (R0 + l/8)*K + 16*chunk (K is a multiple of 128, so the chunk term
    // folds in with an XOR), reduced by 1024*q for the q-th load of a group.
    // MX: every row's chunks are stored in the order cperm (bits 0 and 1 of
    // the chunk index swapped; see the fragment addresses below), which is
    // linear over XOR, so it applies to both XOR terms separately.
    auto cperm = [](int c) { return kMx ? (c & 4) | ((c & 1) << 1) | ((c >> 1) & 1) : c; };
    const int rl = lane >> 3;
    const uint32_t lane_off = (uint32_t)(rl * K) | (uint32_t)(cperm((lane & 7) ^ rl) << 4);
    uint32_t vx[XLOADS], vw[WLOADS];
#pragma unroll
    for (int q = 0; q < XLOADS; ++q) {
        const int grp = wave * XLOADS + q;
        vx[q] = (lane_off ^ (uint32_t)(cperm(grp & 1) << 4)) + (uint32_t)(grp * 8 * K) - 1024u * q;
    }
#pragma unroll
    for (int q = 0; q < WLOADS; ++q) {
        const int grp = wave * WLOADS + q;
        if constexpr (kW4) {
            // E2M1 rows of 64 bytes: a load fills 16 rows; lane l writes slot
            // l%4 of row R0 + l/4, which holds chunk slot ^ swz4(row) with
            // swz4(r) = (r/4) mod 4 = (l/16) mod 4 for R0 a multiple of 16
            const uint32_t off4 = (uint32_t)((lane >> 2) * (K / 2)) | (uint32_t)(((lane & 3) ^ ((lane >> 4) & 3)) << 4);
            vw[q] = off4 + (uint32_t)(grp * 16 * (K / 2)) - 1024u * q;
        } else {
            vw[q] = (lane_off ^ (uint32_t)(cperm(grp & 1) << 4)) + (uint32_t)(grp * 8 * K) - 1024u * q;
        }
    }
    // LDS fragment addresses within a stage: row r, 16-byte chunk c at
    // r*128 + 16*(c ^ swz(r)); this lane reads chunks 2g and 2g+1.
    // The swizzle depends on the row mod 16 only, so subtile i of this wave
    // sits at a fixed distance 2048*i from subtile 0: one base address per
    // 16-byte half, the subtile and stage offsets are ds_read immediates.
    // MX: the scaled 16x16x128 instruction counts a lane's first 16 bytes
    // into scale block g/2 and its last 16 into block 2 + g/2, and applies the
    // scale of lane group j to block j (measured on gfx950).  Any K order
    // inside a block sums alike, so a block only has to hold the two 16-byte
    // chunks of one 32-group of the data: lane group g holds data chunks
    // 4(g/2) + g%2 and that + 2 -- groups 0,1: {0,2},{1,3} (data group 0 in
    // block 0, group 1 in block 2); groups 2,3: {4,6},{5,7} (data groups 2
    // and 3 in blocks 1 and 3) -- and passes the scale of data group
    // mx_grp = (0,2,1,3)[g].  Data chunk c is stored at logical position
    // cperm(c), which turns exactly those chunks into positions 2g and 2g+1:
    // the reads keep the address pattern of the other paths, which has no LDS
    // bank conflicts (reading chunks 4(g/2) + g%2 + {0, 2} directly measured
    // 2e7 conflict cycles per launch).  (The other paths give every 32-group
    // of a row the same scale, and any K order common to both operands sums
    // alike.)
    const int mx_grp = ((g & 1) << 1) | (g >> 1);
    uint32_t xa[2], wa[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = lane & 15;
        const int ch = 2 * g + h;
        xa[h] = (uint32_t)((wm * TM + r) * 128 + ((ch ^ lds_swz(r)) << 4));
        wa[h] = (uint32_t)(W_BASE + (wn * TN + r) * 128 + ((ch ^ lds_swz(r)) << 4));
    }
    // E2M1 W: an FP4 operand lane holds 32 consecutive K of its hardware
    // scale block g (measured: nibble t is K 32g + t, low nibble first, with
    // the scale of lane group g).  Against the X operand's order above that
    // is data group mx_grp: one 16-byte chunk of the row's 64 bytes, read
    // from its swizzled slot mx_grp ^ (r/4 mod 4).
    const uint32_t wa4 = (uint32_t)(W_BASE + (wn * TN + (lane & 15)) * 64 + ((mx_grp ^ (((lane & 15) >> 2) & 3)) << 4));
    // activation scale of row r of the tile at SC + 4r; weight scales at
    // SC + 256*NSA + 4*slot (the first copy)
    // (MX: the row's dword of 4 group bytes; this lane takes byte mx_grp, the
    // 32-group whose chunks it holds.  The dword is read whole: the 4 lanes of
    // a row then read one address, which LDS broadcasts, where byte reads of
    // different bytes of one dword conflict.)
    const uint32_t saa = (uint32_t)(SC_BASE + 4 * (wm * TM + (lane & 15)));
    const uint32_t mx_shift = 8u * (uint32_t)mx_grp;
    // MX: the dword of this lane's column in subtile j of the wave at
    // mx_wcol + 64*j (subtile and stage offsets are immediates)
    const uint32_t mx_wcol = (uint32_t)(SC_BASE + 4 * BM + 4 * (wn * TN + (lane & 15)));
    const bool sa_wave = kMx ? wave < MX_XS_WAVES : wave < NSA;
    // MX: waves 0 .. BM/64-1 load the X scale dwords of 64 tile rows each,
    // the next ones those of 64 tile columns each; in the packed tables the
    // dwords of one K block are consecutive over rows (256 bytes per wave)
    const uint32_t mx_row = (uint32_t)(64 * (sa_wave ? wave : wave - MX_XS_WAVES) + lane);
    const uint32_t sc_voff = kMx ? 4u * mx_row
                                 : (sa_wave ? (uint32_t)(4 * (64 * wave + lane)) : (uint32_t)(4 * lane * KB));
    const uint32_t lds0 = uniform((int)lds_addr(smem));
    // LDS destination of this wave's W loads: its rows in stage s at
    // w_dst + s*w_sstride, or the spare area (every stage) for a wave past them
    const bool w_wave = W_WAVES == NWAVES || wave < W_WAVES;
    const uint32_t w_dst = w_wave ? (uint32_t)(W_BASE + wave * WLOADS * 1024) : (uint32_t)SPARE_BASE;
    const uint32_t w_sstride = w_wave ? (uint32_t)(BN * WROW) : 0u;

    // XCD-aware order: workgroups are dispatched round-robin over the 8 XCDs,
    // so workgroup b of a wave of G lands on XCD b%8.  Give each XCD a run of
    // G/8 consecutive logical tiles (a compact raster patch sharing operand
    // rows in that XCD's L2).
    const int G = gridDim.x;
    // (masked layout: one workgroup per possible tile, no remap)
    const bool remap = MODE != kMasked && (G & 7) == 0;
    const int rounds = (total_tiles + G - 1) / G;

    for (int round = 0; round < rounds; ++round) {
        int t = blockIdx.x;
        if (remap) t = (t & 7) * (G >> 3) + (t >> 3);
        t += round * G;
        if (t >= total_tiles) continue;

        // ---------------- tile decode ----------------
        TileCoord tc;
        if constexpr (MODE == kMasked) {
            // up to 64 experts: the largest first (the tiles' costs follow the counts)
            if (p.E <= 64) {
                if (!decode_tile_masked_by_count<BM, BN>(t, p, masked_m_, tc)) continue;
            } else if (!decode_tile<MODE, BM, BN>(t, p, m_indices_, masked_m_, tc)) {
                continue;
            }
        } else if (MODE == kContiguous && p.pair_cus > 0) {
            decode_tile_paired<BM, BN>(t, p, pair_ent, pair_sh, tc);
        } else if (!decode_tile<MODE, BM, BN>(t, p, m_indices_, masked_m_, tc)) {
            continue;
        }
        const int64_t row0 = tc.row0, row_end = tc.row_end, n0 = tc.n0;
        const int expert = tc.expert;
        const uint8_t* wq = wq_;
        const float* sb = sb_;
        if constexpr (MODE != kDense) {
            wq += (int64_t)expert * N * K;
            sb += (int64_t)expert * (N / 128) * KB;
        }
        const int rows_valid = (int)min((int64_t)BM, row_end - row0);
        const int cols_valid = (int)min((int64_t)BN, N - n0);

        // Buffer resources of this tile: rows past the valid range read zeros.
        const i32x4 xr = make_rsrc(xq_ + row0 * K, (uint32_t)(rows_valid * K));
        const int64_t KW = kW4 ? K / 2 : K;   // bytes per W row
        const i32x4 wr = make_rsrc(wq + n0 * KW, (uint32_t)(cols_valid * KW));
        const float* sa_row0 = sa_ + row0;
        // Weight scales: lane l of a wave's scale load fetches block row
        // nb0 + l; rows past the last weight block read zero.
        const int nb0 = (int)(n0 >> 7);
        const int nbl = (int)min((int64_t)(BN / 128 + 2), (N + 127) / 128 - nb0);
        // This wave's scale load, as a base that advances adv bytes per K
        // block, an soffset of sstep bytes per K block and a byte range.
        // (MX: the tile's rows, or columns, of the packed [K/128][M] or
        // [K/128][N] dword tables, advancing one table row per K block)
        const uint64_t sc_base = uniform_u64(
            kMx ? (sa_wave ? (uint64_t)(reinterpret_cast<const uint32_t*>(sa_) + row0)
                           : (uint64_t)(reinterpret_cast<const uint32_t*>(sb_) + n0))
                : (sa_wave ? (uint64_t)sa_row0 : (uint64_t)(sb + (int64_t)nb0 * KB)));
        const uint32_t sc_adv = kMx ? (uint32_t)(4 * (sa_wave ? p.M : N))
                                    : (sa_wave ? (uint32_t)(4 * p.M) : 0u);
        const int sc_step = (kMx || sa_wave) ? 0 : 4;
        const uint32_t sc_rec = uniform(
            kMx ? (sa_wave ? (int)(4 * rows_valid)
                           : (wave < MX_XS_WAVES + MX_WS_WAVES ? (int)(4 * cols_valid) : 0))
                : (sa_wave ? (int)(4 * rows_valid) : (int)(4 * nbl * KB)));
        // LDS slot of each subtile's weight block (the last block for
        // subtiles past N, whose columns are never stored)
        uint32_t sb_slot[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            const int64_t n = n0 + wn * TN + 16 * j;
            if constexpr (!kMx)   // (MX: mx_wcol)
                sb_slot[j] = (uint32_t)(SC_BASE + 256 * NSA + 4 * ((int)((n < N ? n : N - 1) >> 7) - nb0));
        }
        // split scales: subtiles 0 .. jb-1 of this wave lie in the weight block
        // of slot sb_slot[0], the others in the next one (for a wave past N
        // both slots hold a loaded scale or zero, and its columns are not stored)
        int jb = FJ;
        if constexpr (kSplitSb) {
            const int nw = (int)((n0 + wn * TN) & 127);
            jb = nw == 0 ? FJ : min(FJ, (128 - nw) / 16);
        }

        // Issue the loads of K block kb into stage s.  Past the last block the
        // resources get an empty range, so the loads are discarded by the
        // range check without a branch (the loop body stays one basic block).
        // A stage is issued as NPIECE single loads (X rows, W rows, scales)
        // so that they can be spread between the MFMAs of a step.
        struct StageLoads {
            uint32_t xm0, wm0, sm0;
            i32x4 xr, wr, sr;
            int koff, wkoff, soff;
        };
        auto stage_loads = [&](int kb, auto bufc) {
            constexpr uint32_t s = decltype(bufc)::value;
            // all ones for a real block, zero past the last one (only the
            // ranges are cleared: nothing outside an empty range is read)
            const int live = -(int)(kb < KB);
            StageLoads L;
            L.xm0 = lds0 + s * BM * 128 + (uint32_t)(wave * XLOADS * 1024);
            L.wm0 = lds0 + w_dst + s * w_sstride;
            L.sm0 = lds0 + SC_BASE + s * NWAVES * 256 + (uint32_t)(wave * 256);
            L.xr = xr;
            L.wr = wr;
            L.xr[2] = xr[2] & live;
            L.wr[2] = wr[2] & live;
            // scales: activation row kb of sA, or weight-block column kb of sB
            const uint64_t scb = sc_base + (uint64_t)(uint32_t)kb * sc_adv;
            L.sr = i32x4{(int)(uint32_t)scb, (int)(uint32_t)(scb >> 32) & 0xFFFF, (int)sc_rec & live,
                         0x00020000};
            L.koff = kb * 128;
            L.wkoff = kb * WROW;
            L.soff = kb * sc_step;
            return L;
        };
        auto issue_piece = [&](const StageLoads& L, auto pc) {
            constexpr int P = decltype(pc)::value;
            if constexpr (P < XLOADS) dma_lds16_one<P>(L.xm0, vx[P], L.xr, L.koff);
            else if constexpr (P < XLOADS + WLOADS) dma_lds16_one<P - XLOADS>(L.wm0, vw[P - XLOADS], L.wr, L.wkoff);
            else dma_lds4(L.sm0, sc_voff, L.sr, L.soff);
        };

        // ---------------- K loop ----------------
        // One operand is held in registers for a whole K block (C resident
        // fragments); the other streams through one 16-row subtile at a time
        // (R rows per block).  The operand with fewer subtiles per wave is the
        // resident one, which keeps the fragment registers low.  One software
        // pipeline runs over the streamed rows, global row g = kb*R + r,
        // across K blocks:
        //   * the fragment and scale of row g are read at row g-2;
        //   * the barrier of block kb sits just before row R-2 of block kb:
        //     by then every wave has finished its reads of block kb and its
        //     loads of block kb+1 have landed; after it, block kb's buffer
        //     takes the loads of block kb+STAGES and block kb+1 may be read;
        //   * the resident fragments and scales of block kb+1 are read during
        //     the last row of block kb, each fragment right after its last MFMA;
        //   * the loads of the blocks ahead are spread over the rows;
        //   * row g's partials are promoted during row g+1.
        // Promotion scale of a subtile: the streamed row's scale times the
        // resident fragment's scale (sA x sB in either orientation).
        constexpr int R = kStreamW ? FJ : FI;   // streamed rows per K block
        constexpr int C = kStreamW ? FI : FJ;   // resident fragments
        static_assert(STAGES >= 2 && R >= 2, "pipeline of at least two stages over at least two subtile rows");
        constexpr int RB = R - 2;   // row before which the barrier of a block sits
        auto read_x = [&](int buf, int i) { return lds_frag(smem + buf * BM * 128 + 2048 * i, xa[0], xa[1]); };
        // (wa already holds the W region's base)
        auto read_w = [&](int buf, int j) {
            if constexpr (kW4) {
                // 16 bytes (32 E2M1 values); the instruction reads 4 registers
                const i32x2 lo = *reinterpret_cast<const i32x2*>(smem + buf * BN * 64 + 1024 * j + wa4);
                const i32x2 hi = *reinterpret_cast<const i32x2*>(smem + buf * BN * 64 + 1024 * j + wa4 + 8);
                return i32x8{lo[0], lo[1], hi[0], hi[1], 0, 0, 0, 0};
            } else {
                return lds_frag(smem + buf * BN * 128 + 2048 * j, wa[0], wa[1]);
            }
        };
        auto read_sa = [&](int buf, int i) -> ScaleT {
            if constexpr (kMx)
                return (int)__builtin_amdgcn_ubfe(
                    *reinterpret_cast<const uint32_t*>(smem + buf * NWAVES * 256 + saa + 64 * i), mx_shift, 8);
            else return *reinterpret_cast<const float*>(smem + buf * NWAVES * 256 + saa + 64 * i);
        };
        auto read_sb = [&](int buf, int j) -> ScaleT {
            if constexpr (kMx)
                return (int)__builtin_amdgcn_ubfe(
                    *reinterpret_cast<const uint32_t*>(smem + buf * NWAVES * 256 + mx_wcol + 64 * j), mx_shift, 8);
            else return *reinterpret_cast<const float*>(smem + buf * NWAVES * 256 + sb_slot[j]);
        };
        // the E8M0 operand of the scaled MFMA
        auto e8m0 = [&](ScaleT v) -> int {
            if constexpr (kMx) return v;
            else return e8m0_of(v);
        };
        auto read_row = [&](int buf, int r) {
            if constexpr (kStreamW) return read_w(buf, r);
            else return read_x(buf, r);
        };
        auto read_row_scale = [&](int buf, int r) -> ScaleT {
            if constexpr (kSplitSb) return 0.f;   // the block's two products serve every row
            else if constexpr (kStreamW) return read_sb(buf, r);
            else return read_sa(buf, r);
        };
        // split scales: the two weight-block scales of this wave
        auto read_sb2 = [&](int buf, float (&v)[2]) {
            v[0] = *reinterpret_cast<const float*>(smem + buf * NWAVES * 256 + sb_slot[0]);
            v[1] = *reinterpret_cast<const float*>(smem + buf * NWAVES * 256 + sb_slot[0] + 4);
        };
        auto read_res = [&](int buf, int c) {
            if constexpr (kStreamW) return read_x(buf, c);
            else return read_w(buf, c);
        };
        auto read_res_scales = [&](int buf, ScaleT (&v)[C]) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                if constexpr (kStreamW) v[c] = read_sa(buf, c);
                else if (kUniformSb && !kMx && c > 0) v[c] = v[0];
                else v[c] = read_sb(buf, c);
            }
        };
        // The loads of a block go out over the first WIN of the R rows that
        // follow the barrier which frees their buffer (window positions
        // 0 .. WIN-1); the remaining rows before the next barrier leave time
        // for the last ones to land (measured: 3/4 of the rows is best).
        constexpr int WIN = R >= 4 ? (3 * R) / 4 : R;
        auto issue_window = [&](const StageLoads& L, auto posc) {
            constexpr int pos = decltype(posc)::value;
            __builtin_amdgcn_sched_barrier(0x0006);
            static_for<NPIECE>([&](auto pc) {
                constexpr int P = decltype(pc)::value;
                if constexpr (P * WIN / NPIECE == pos) issue_piece(L, pc);
            });
            __builtin_amdgcn_sched_barrier(0x0006);
        };

        f32x4 acc[FI][FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};
        // accumulator of streamed row r, resident fragment c
        auto accr = [&](int r, int c) -> f32x4& {
            if constexpr (kStreamW) return acc[c][r];
            else return acc[r][c];
        };

        // The K loop, specialised on JB: with split scales, the streamed rows
        // 0 .. JB-1 take the first weight block's products (JB = 0 otherwise).
        // FV: the streamed rows (16-row X subtiles) of this wave that hold
        // valid rows; the masked layout skips the multiplies of the others.
        auto kloop = [&](auto jbc, auto fvc) {
        constexpr int JB = decltype(jbc)::value;
        constexpr int FV = decltype(fvc)::value;
        // Prologue: blocks 0 .. STAGES-2 in full, all in flight together; once
        // block 0 has landed (for every wave), the first two window positions
        // of block STAGES-1; then the reads of block 0 that the pipeline
        // expects.
        // All waves are done with the previous tile's buffers.  No wait for the
        // vector-memory counter here: it also counts the previous tile's output
        // stores, and the waits below are counts of this wave's loads issued
        // after the one waited for, which loads complete in order.  Each wave
        // refills only its own rows of a buffer, after its own earlier loads
        // into them (the discarded ones past the previous tile's last block).
        lds_barrier();
        static_for<STAGES - 1>([&](auto sc) {
            constexpr int b = decltype(sc)::value;
            const StageLoads Lb = stage_loads(b, std::integral_constant<int, b>{});
            static_for<NPIECE>([&](auto pc) { issue_piece(Lb, pc); });
        });
        wait_vmcnt<(STAGES - 2) * NPIECE>();   // block 0: blocks 1 .. STAGES-2 may fly
        lds_barrier();
        {
            const StageLoads Ll = stage_loads(STAGES - 1, std::integral_constant<int, STAGES - 1>{});
            issue_window(Ll, std::integral_constant<int, 0>{});
            issue_window(Ll, std::integral_constant<int, 1>{});
        }
        i32x8 res[C];
#pragma unroll
        for (int c = 0; c < C; ++c) res[c] = read_res(0, c);
        ScaleT rs_cur[C], rs_prev[C];
        read_res_scales(0, rs_cur);
#pragma unroll
        for (int c = 0; c < C; ++c) rs_prev[c] = ScaleT{};
        // fragments and scales of the next two streamed rows (g, g+1)
        i32x8 fr0 = read_row(0, 0), fr1 = read_row(0, 1);
        ScaleT sr0 = read_row_scale(0, 0), sr1 = read_row_scale(0, 1);
        // the partials of the row before (none yet: zeros promote to nothing)
        f32x4 prev[C];
#pragma unroll
        for (int c = 0; c < C; ++c) prev[c] = f32x4{0.f, 0.f, 0.f, 0.f};
        ScaleT st_prev{};
        // split scales: this block's weight-block scales, the products
        // sA(c) x sB(first / second block), and the products of the previous
        // block's last row
        float sb2_cur[2], pr[2][C], plast[C];
        if constexpr (kSplitSb) {
            read_sb2(0, sb2_cur);
#pragma unroll
            for (int c = 0; c < C; ++c) plast[c] = 0.f;
        }
        auto promote_p = [&](int rp, const float (&pv)[C]) {
#pragma unroll
            for (int c = 0; c < C; ++c)
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) accr(rp, c)[r2] = fmaf(pv[c], prev[c][r2], accr(rp, c)[r2]);
        };

        // promotion of the previous row (partials prev, row rp of the block
        // whose resident scales are rsv)
        auto promote = [&](int rp, const float (&rsv)[C]) {
#pragma unroll
            for (int c = 0; c < C; ++c) {
                const float sc = st_prev * rsv[c];
#pragma unroll
                for (int r2 = 0; r2 < 4; ++r2) accr(rp, c)[r2] = fmaf(sc, prev[c][r2], accr(rp, c)[r2]);
            }
        };

        auto step = [&](int kb, auto bufc) {
            constexpr int BUF = decltype(bufc)::value;           // buffer of block kb
            constexpr int NBUF = (BUF + 1) % STAGES;             // of block kb+1
            // loads of block kb+STAGES-1 (window positions 2 .. R-1, into the
            // buffer of block kb-1) and of block kb+STAGES (positions 0, 1,
            // after the barrier, into this block's buffer)
            const StageLoads L1 =
                stage_loads(kb + STAGES - 1, std::integral_constant<int, (BUF + STAGES - 1) % STAGES>{});
            const StageLoads L2 = stage_loads(kb + STAGES, std::integral_constant<int, BUF>{});
            ScaleT rs_next[C];
            float sb2_next[2];
            // E8M0 exponents of the resident scales (scaled-MFMA path)
            int rse[C];
            if constexpr (kScaledMfma) {
#pragma unroll
                for (int c = 0; c < C; ++c) rse[c] = e8m0(rs_cur[c]);
            }
            static_for<R>([&](auto rc) {
                constexpr int r = decltype(rc)::value;
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (r == RB) {
                    // every read of block kb is done (lgkm) and this wave's
                    // loads of block kb+1 have landed (vm: only those of blocks
                    // kb+2 .. kb+STAGES-1 may still fly); then publish
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    wait_vmcnt<(STAGES - 2) * NPIECE>();
                    lds_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                }
                const i32x8 fc = fr0;
                const ScaleT st_c = sr0;
                // reads two rows ahead: this block, or the next one after the barrier
                i32x8 fn;
                ScaleT sn;
                if constexpr (r + 2 < R) {
                    fn = read_row(BUF, r + 2);
                    sn = read_row_scale(BUF, r + 2);
                } else {
                    fn = read_row(NBUF, r + 2 - R);
                    sn = read_row_scale(NBUF, r + 2 - R);
                }
                fr0 = fr1;
                fr1 = fn;
                sr0 = sr1;
                sr1 = sn;
                if constexpr (r == R - 1) {
                    read_res_scales(NBUF, rs_next);
                    if constexpr (kSplitSb) read_sb2(NBUF, sb2_next);
                }
                // loads of the blocks ahead
                if constexpr (r < RB) issue_window(L1, std::integral_constant<int, r + 2>{});
                else issue_window(L2, std::integral_constant<int, r - RB>{});

                if constexpr (kScaledMfma) {
                    const int ste = e8m0(st_c);
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        // operand A is the W fragment, B the X fragment
                        // operand format of A (W): 0 E4M3, 4 E2M1; B (X) is E4M3
                        constexpr int kFmtA = kW4 ? 4 : 0;
                        if constexpr (r >= FV) {
                            // a subtile past the valid rows (masked): nothing to multiply
                        } else if constexpr (kStreamW)
                            accr(r, c) = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                fc, res[c], accr(r, c), kFmtA, 0, 0, ste, 0, rse[c]);
                        else
                            accr(r, c) = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                res[c], fc, accr(r, c), kFmtA, 0, 0, rse[c], 0, ste);
                        if constexpr (r == R - 1) res[c] = read_res(NBUF, c);
                    }
                } else {
                    f32x4 cur[C];
#pragma unroll
                    for (int c = 0; c < C; ++c) {
                        if constexpr (r >= FV) {
                            // past the valid rows (masked): nothing to multiply
                        } else if constexpr (kStreamW)
                            cur[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                fc, res[c], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                        else
                            cur[c] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                res[c], fc, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                        if constexpr (r == R - 1) res[c] = read_res(NBUF, c);
                    }
                    // the previous row: row r-1 of this block, or the last
                    // row of the previous block (with that block's scales)
                    if constexpr (kSplitSb) {
                        // this block's products, formed once its scales have
                        // surely arrived (read during the previous block's last row)
                        if constexpr (r == 1) {
#pragma unroll
                            for (int h = 0; h < 2; ++h)
#pragma unroll
                                for (int c = 0; c < C; ++c)
                                    pr[h][c] = rs_cur[c] * sb2_cur[h];
                        }
                        if constexpr (r == 0) promote_p(R - 1, plast);
                        else promote_p(r - 1, pr[r - 1 < JB ? 0 : 1]);
                    } else {
                        // (rows past the valid ones, masked: no partials to promote)
                        if constexpr (r == 0) {
                            if constexpr (R - 1 < FV) promote(R - 1, rs_prev);
                        } else if constexpr (r - 1 < FV) {
                            promote(r - 1, rs_cur);
                        }
                    }
                    if constexpr (r < FV) {
#pragma unroll
                        for (int c = 0; c < C; ++c) prev[c] = cur[c];
                        st_prev = st_c;
                    }
                    // each MFMA of this row preceded by the promotion FMAs of
                    // the subtile whose partials its result replaces (and the
                    // scale products)
                    if constexpr (r < FV) {
                        static_for<C>([&](auto qc) {
                            constexpr int n = kSplitSb ? 4 : (decltype(qc)::value == 0 || kStreamW ? 5 : 4);
                            __builtin_amdgcn_sched_group_barrier(0x002, n, 0);
                            __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        });
                    }
                }
            });
            __builtin_amdgcn_sched_barrier(0);
#pragma unroll
            for (int c = 0; c < C; ++c) {
                rs_prev[c] = rs_cur[c];
                rs_cur[c] = rs_next[c];
            }
            if constexpr (kSplitSb) {
#pragma unroll
                for (int c = 0; c < C; ++c) plast[c] = pr[R - 1 < JB ? 0 : 1][c];
                sb2_cur[0] = sb2_next[0];
                sb2_cur[1] = sb2_next[1];
            }
        };
        // K loop unrolled by the ring of buffers (straight-line body), then the tail.
        int kb = 0;
        for (; kb + STAGES <= KB; kb += STAGES)
            static_for<STAGES>([&](auto sc) { step(kb + decltype(sc)::value, sc); });
        static_for<STAGES - 1>([&](auto sc) {
            if (kb + decltype(sc)::value < KB) step(kb + decltype(sc)::value, sc);
        });
        // drain: the last row's partials
        if constexpr (kSplitSb) promote_p(R - 1, plast);
        else if constexpr (!kScaledMfma && R - 1 < FV) promote(R - 1, rs_prev);
        };
        if constexpr (kSplitSb) {
            // one copy of the loop per boundary position (wave-uniform)
            static_for<FJ>([&](auto jc) {
                if (jb == decltype(jc)::value + 1)
                    kloop(std::integral_constant<int, decltype(jc)::value + 1>{}, std::integral_constant<int, R>{});
            });
        } else {
            if constexpr (MODE == kMasked) {
                const int fv = uniform(min(max(rows_valid - wm * TM + 15, 0) / 16, R));
                static_for<R + 1>([&](auto fc) {
                    if (fv == decltype(fc)::value) kloop(std::integral_constant<int, 0>{}, fc);
                });
            } else {
                kloop(std::integral_constant<int, 0>{}, std::integral_constant<int, R>{});
            }
        }
        // (the loads issued past the last block were discarded; they retire in
        // order before the next tile's loads, and the kernel's end waits for them)

        const int g4 = 4 * g;
        if constexpr (QOUT) {
            // ---------------- epilogue: E4M3 + 1x128 scales along N ----------------
            // A 128-column group of a row spans this wave's 64 columns and
            // those of its neighbour wn^1.  Row maximum over the wave's
            // columns: 16 values per lane, then across the 4 lanes of the
            // row (lanes l, l^16, l^32, l^48); the two waves of a group meet
            // in LDS.  Scale and codes as the 1x128 quantizer defines them,
            // applied to the FP32 accumulator.
            float* qa = reinterpret_cast<float*>(smem + QA_BASE);
            float own[FI];
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                float a = 0.f;
#pragma unroll
                for (int j = 0; j < FJ; ++j)
#pragma unroll
                    for (int r2 = 0; r2 < 4; ++r2) a = fmaxf(a, fabsf(acc[i][j][r2]));
                a = fmaxf(a, __shfl_xor(a, 16));
                a = fmaxf(a, __shfl_xor(a, 32));
                own[i] = a;
                if (g == 0) qa[wn * BM + wm * TM + 16 * i + (lane & 15)] = a;
            }
            __syncthreads();
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const int mloc = wm * TM + 16 * i + (lane & 15);
                const int64_t m = row0 + mloc;
                if (mloc >= rows_valid) continue;
                const float s = group_scale(fmaxf(own[i], qa[(wn ^ 1) * BM + mloc]), kPow2);
#pragma unroll
                for (int j = 0; j < FJ; ++j) {
                    const int64_t n = n0 + wn * TN + 16 * j + g4;   // N % 128 == 0: n < N covers n+3
                    if (n < N)
                        *reinterpret_cast<uint32_t*>(p.yq + m * N + n) =
                            cvt_e4m3x4(acc[i][j][0] / s, acc[i][j][1] / s, acc[i][j][2] / s, acc[i][j][3] / s);
                }
                const int64_t nw = n0 + wn * TN;
                if (g == 0 && (wn & 1) == 0 && nw < N) p.sy[(nw >> 7) * p.M + m] = s;
            }
            continue;
        }
        // ---------------- epilogue: BF16 (RNE), predicated stores ----------------
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int mloc = wm * TM + 16 * i + (lane & 15);
            const int64_t m = row0 + mloc;
            bool ok = mloc < rows_valid;
            if constexpr (MODE == kContiguous)
                if (ok) ok = m_indices_[m] == expert;
            if (!ok) continue;
            uint16_t* yrow = y_ + m * N;
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int64_t n = n0 + wn * TN + 16 * j + g4;
                const uint32_t lo = pack_bf16x2(acc[i][j][0], acc[i][j][1]);
                const uint32_t hi = pack_bf16x2(acc[i][j][2], acc[i][j][3]);
                if ((N & 3) == 0 && n + 3 < N) {
                    *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
                } else {
                    if (n < N) yrow[n] = (uint16_t)(lo & 0xFFFF);
                    if (n + 1 < N) yrow[n + 1] = (uint16_t)(lo >> 16);
                    if (n + 2 < N) yrow[n + 2] = (uint16_t)(hi & 0xFFFF);
                    if (n + 3 < N) yrow[n + 3] = (uint16_t)(hi >> 16);
                }
            }
        }
    }
    // The last stages issued were discarded loads; let them retire before the
    // workgroup's LDS is released.
    wait_vmcnt<0>();
}

}  // namespace fp8k
