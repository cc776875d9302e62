// kernels_exact.h -- block-scaled E4M3 NT GEMM for gfx950 with exact block
// partials: the default path of libfp8gemm.so.
//
// Computes Y = X * W^T (BF16 out) with X (M,K) E4M3 + one FP32 scale per 1x128
// tile of a row and W (N,K) E4M3 + one FP32 scale per 128x128 block:
//   Y[m][n] = sum_kb sa[kb][m] * sb[n/128][kb] * P_kb[m][n],
//   P_kb[m][n] = sum_{k in block kb} X[m][k] * W[n][k]
// (tcgen05 page, section 6.1: the block-scaled product; DeepGEMM page,
// section "主循环骨架": each 128-K block partial is multiplied by sA*sB and
// added to a full-precision accumulator; section "细粒度缩放在 GEMM 层面引爆的
// 两个问题": the promotion exists so that the sum is accumulated at full
// precision).
//
// gfx950 mapping
//   * Exact products.  Every E4M3 value is an FP16 value (4 significant bits,
//     2^-9 .. 448), so the operands are widened with the hardware converter at
//     scale 1 and multiplied by v_mfma_f32_32x32x16_f16, whose products are
//     exact in FP32 and whose sums are FP32-accurate (measured on every pair of
//     E4M3 codes: within 3 * 2^-24 * sum |products|).  The FP8 matrix
//     instructions of gfx950 truncate small products inside each group of 8
//     (they remain available as the opt-in FP8_FLAG_FAST_ACCUM path,
//     kernels_gemm.h).  The 32x32x16 form runs at the full FP16 rate; the
//     16x16x32 form measured at about half of it.
//   * Promotion without partial registers.  The FP32 accumulator of a 32x32
//     subtile is kept in units of the current block's scale product
//     s_kb = sa * sb: before the first MFMA of block kb it is multiplied by
//     s_{kb-1} / s_kb, then the block's MFMAs add P_kb to it, and after the
//     last block it is multiplied by s_last.  So acc * s_kb equals
//     sum_{j <= kb} s_j P_j after every block, the DeepGEMM promotion, with
//     one VALU multiply per accumulator value and block and no second set of
//     accumulators.  With power-of-two scales (FP8_FLAG_UE8M0) the factors
//     are exact exponent shifts (v_ldexp_f32).
//   * Subtiles.  A wave owns TM x TN = FI x FJ subtiles of 32x32; W is the
//     MFMA A operand and X the B operand, so lane l of a subtile holds one
//     output row m (column l%32 of the result) and 16 columns n, all inside
//     one 128-row weight block: one sA and one sB per lane and subtile.
//   * K order.  A 128-K block is 8 MFMA steps of 16.  In step s lane l takes
//     the 8 bytes 64*(l/32) + 8*s .. +7 of its row's K block: lane group l/32
//     covers one half of the block over the 8 steps.  The same order serves
//     both operands, and a dot product does not depend on the order of K.
//   * LDS.  Operands reach LDS as E4M3 with buffer_load_dwordx4 ... lds (no
//     VGPR staging), through per-tile buffer resources whose range ends at the
//     last valid row (rows past it read zeros).  Each tile row is one
//     128-byte K block; its eight 16-byte chunks are XOR-swizzled
//     (gemm_common.h: lds_swz).  A lane reads 16 bytes (two steps) per
//     subtile with one ds_read_b128; the 16 lanes of each quarter-wave read
//     16 rows at one logical chunk, which the swizzle spreads over all banks.
//   * A ring of STAGES LDS buffers; each wave waits on its own vector-memory
//     counter for the oldest stage, then one barrier per K block publishes it
//     and frees the buffer of the block before.  The loads of a block are
//     spread between the MFMA steps.
//   * Persistent grid with the XCD-aware grouped raster order and the grouped
//     tile walks of gemm_common.h.
//   * Masked layout: one workgroup per possible tile (the hardware dispatcher
//     balances tiles of unequal cost), and each wave multiplies only its
//     32-row subtiles that hold valid rows (DeepGEMM page, "分组 GEMM 的两种
//     布局": the masked layout computes the valid positions only), so a
//     tile's cost follows its expert's count in steps of 32 rows; the tiles
//     are walked largest expert first (gemm_common.h), so the dispatcher
//     starts the longest ones first.  The tile body (kernels_exact_tile.inc)
//     is instantiated once per number of valid subtiles.
#pragma once

#include "gemm_common.h"

namespace fp8k {

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE, bool POW2, int STAGES, bool QOUT = false>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_exact_kernel(
    const uint8_t* __restrict__ xq_, const float* __restrict__ sa_, const uint8_t* __restrict__ wq_,
    const float* __restrict__ sb_, uint16_t* __restrict__ y_, const int32_t* __restrict__ m_indices_,
    const int32_t* __restrict__ masked_m_, GemmParams p) {
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int TM = BM / WAVES_M;    // wave tile rows (m)
    constexpr int TN = BN / WAVES_N;    // wave tile columns (n)
    constexpr int FI = TM / 32;         // 32x32 subtiles along m
    constexpr int FJ = TN / 32;         // ... along n
    // A stage is BM/8 X pieces and BN/8 W pieces of 1 KB (8 rows of one K
    // block each), dealt to the waves round-robin: X piece q of wave w is
    // 8-row group q*NWAVES + w of the X tile, W piece q likewise of the W
    // tile.  A wave whose group lies past the tile loads nothing real (an
    // empty range) into a spare area, so every wave issues the same number of
    // loads and one vmcnt target serves all.
    constexpr int NXP = BM / 8, NWP = BN / 8;
    constexpr int XPER = (NXP + NWAVES - 1) / NWAVES, WPER = (NWP + NWAVES - 1) / NWAVES;
    constexpr int PER = XPER + WPER;
    constexpr bool kPad = XPER * NWAVES > NXP || WPER * NWAVES > NWP;
    constexpr int NPIECE = PER + 1;     // + one scale load
    // scales of a stage: waves 0 .. NSA-1 load the activation scales of the
    // tile's rows (64 each); every other wave loads a copy of the weight
    // scales of the tile's 128-row weight blocks (one per lane)
    constexpr int NSA = BM / 64;
    constexpr int W_BASE = STAGES * BM * 128;
    constexpr int SC_BASE = W_BASE + STAGES * BN * 128;
    constexpr int SPARE_BASE = SC_BASE + STAGES * NWAVES * 256;
    constexpr int LDS_BYTES = SPARE_BASE + (kPad ? 1024 : 0);
    constexpr int NP = 4;               // 16-byte reads (pairs of MFMA steps) per K block
    constexpr int RB = NP - 1;          // the pair before which a block's barrier sits
    constexpr int WIN = 3;              // window positions over which a block's loads go out
    static_assert(TM % 32 == 0 && TN % 32 == 0, "wave tile: whole 32x32 subtiles");
    static_assert(NWAVES % 2 == 0, "pieces of one wave share the swizzle parity");
    static_assert(BM % 64 == 0 && NSA < NWAVES, "activation scales: 64 rows per wave, one wave left for sB");
    static_assert(BN / 128 + 2 <= 64, "one scale load covers the tile's weight blocks");
    static_assert(STAGES >= 2 && LDS_BYTES <= 160 * 1024, "LDS holds the stage ring");
    static_assert((STAGES - 2) * NPIECE <= 63 && PER <= 16, "vmcnt range");
    static_assert(!QOUT || (MODE == kDense && TN == 128 && BN % 128 == 0),
                  "quantized output: a 128-column group per wave");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[LDS_BYTES];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    // Wave rows and columns.  Masked layout: wave w takes row w / WAVES_N and
    // column w % WAVES_N, so that with WAVES_N = 4 the two waves sharing a
    // SIMD (w mod 4) own different rows; a tile whose valid rows end early
    // then still gives every SIMD the same share of the multiplies.
    const int wm = MODE == kMasked ? wave / WAVES_N : wave % WAVES_M;
    const int wn = MODE == kMasked ? wave % WAVES_N : wave / WAVES_M;
    const int64_t K = p.K;
    const int KB = (int)(K / 128);
    const int64_t N = p.N;
    const int h = lane >> 5;            // K half of the block this lane covers
    const int r32 = lane & 31;          // row of a 32-row subtile

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

    // ---- per-lane constants ----
    // DMA piece of 8-row group f: lane l writes slot l%8 of row 8f + l/8,
    // which holds logical chunk (l%8) ^ lds_swz(8f + l/8) = (l%8) ^ (l/8) ^ (f%2);
    // source: (8f + l/8)*K + 16*chunk within the tile's rows.  Pieces 0 ..
    // XPER-1 of a wave are X groups, the others W groups.
    // With NWAVES even, group (q*NWAVES + w) has the parity of w: piece q's
    // source offset is voff0 + q*8*NWAVES*K and its LDS offset
    // ldsw + q*NWAVES*1024 within its operand's stage.
    const int rl = lane >> 3;
    const uint32_t voff0 = (uint32_t)((8 * wave + rl) * K) + (uint32_t)(((lane & 7) ^ rl ^ (wave & 1)) << 4);
    const uint32_t qstep = uniform((int)(8 * NWAVES * K));
    // fragment addresses within a stage: row r of a subtile, logical chunk
    // 4h + pr at slot (4h + pr) ^ lds_swz(r); subtile and stage offsets are
    // ds_read immediates (the swizzle depends on r mod 16 only)
    uint32_t xa[NP], wa[NP];
#pragma unroll
    for (int pr = 0; pr < NP; ++pr) {
        const uint32_t slot = (uint32_t)(((4 * h + pr) ^ lds_swz(r32)) << 4);
        xa[pr] = (uint32_t)((wm * TM + r32) * 128) + slot;
        wa[pr] = (uint32_t)(W_BASE + (wn * TN + r32) * 128) + slot;
    }
    uint32_t saa = (uint32_t)(SC_BASE + 4 * (wm * TM + r32));   // + 128*a per subtile
    const bool sa_wave = wave < NSA;
    const uint32_t lds0 = uniform((int)lds_addr(smem));
    const uint32_t ldsw = lds0 + (uint32_t)(wave * 1024);

    // XCD-aware order: workgroup b of a dispatch wave of G lands on XCD b%8;
    // each XCD gets a run of G/8 consecutive logical tiles.
    const int G = gridDim.x;
    // (Masked layout: one workgroup per possible tile, so the hardware
    // dispatcher balances tiles of unequal cost; no remap.)
    const bool remap = MODE != kMasked && (G & 7) == 0;
    const int rounds = (total_tiles + G - 1) / G;

    for (int round = 0; round < rounds; ++round) {
        int t = blockIdx.x;
        if (remap) t = (t & 7) * (G >> 3) + (t >> 3);
        t += round * G;
        if (t >= total_tiles) continue;

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
        const int64_t row0 = tc.row0, n0 = tc.n0;
        const int expert = tc.expert;
        const uint8_t* wq = wq_;
        const float* sb = sb_;
        if constexpr (MODE != kDense) {
            wq += (int64_t)expert * N * K;
            sb += (int64_t)expert * (N / 128) * KB;
        }
        const int rows_valid = (int)min((int64_t)BM, tc.row_end - row0);
        const int cols_valid = (int)min((int64_t)BN, N - n0);

        // buffer resources: rows past the valid range read zeros
        const i32x4 xr = make_rsrc(xq_ + row0 * K, (uint32_t)(rows_valid * K));
        const i32x4 wr = make_rsrc(wq + n0 * K, (uint32_t)(cols_valid * K));
        const int nb0 = (int)(n0 >> 7);
        const int nbl = (int)min((int64_t)(BN / 128 + 2), (N + 127) / 128 - nb0);
        // this wave's scale load: a base advancing adv bytes per K block, an
        // soffset of sstep bytes per K block and a byte range
        const uint64_t sc_base = uniform_u64(sa_wave ? (uint64_t)(sa_ + row0) : (uint64_t)(sb + (int64_t)nb0 * KB));
        const uint32_t sc_adv = sa_wave ? (uint32_t)(4 * p.M) : 0u;
        const int sc_step = sa_wave ? 0 : 4;
        const uint32_t sc_rec = uniform(sa_wave ? (int)(4 * rows_valid) : (int)(4 * nbl * KB));
        const uint32_t sc_voff = sa_wave ? (uint32_t)(4 * (64 * wave + lane)) : (uint32_t)(4 * lane * KB);
        // LDS slot of each W subtile's weight-block scale (the last block for
        // subtiles past N, whose columns are never stored)
        uint32_t sb_slot[FJ];
#pragma unroll
        for (int b = 0; b < FJ; ++b) {
            const int64_t n = n0 + wn * TN + 32 * b;
            sb_slot[b] = (uint32_t)(SC_BASE + 256 * NSA + 4 * ((int)((n < N ? n : N - 1) >> 7) - nb0));
        }

        // Loads of K block kb into stage s: the ranges are cleared past the
        // last block, so the loads are issued without a branch and discarded.
        struct StageLoads {
            int kb, s;
        };
        auto stage_loads = [&](int kb, int s) FP8K_INLINE { return StageLoads{kb, s}; };
        auto issue_piece = [&](const StageLoads& L, auto pc) FP8K_INLINE {
            constexpr int P = decltype(pc)::value;
            const int live = -(int)(L.kb < KB);
            if constexpr (P < PER) {
                constexpr bool isx = P < XPER;
                constexpr int q = isx ? P : P - XPER;
                constexpr uint32_t stride = isx ? BM * 128 : BN * 128;
                i32x4 r = isx ? xr : wr;
                r[2] &= live;
                uint32_t dst = ldsw + (uint32_t)((isx ? 0 : W_BASE) + q * NWAVES * 1024) + (uint32_t)L.s * stride;
                if constexpr (q * NWAVES + NWAVES > (isx ? NXP : NWP)) {
                    // waves whose group lies past the tile: empty range, spare area
                    if (q * NWAVES + wave >= (isx ? NXP : NWP)) {
                        r[2] = 0;
                        dst = lds0 + SPARE_BASE;
                    }
                }
                dma_lds16_one<0>(dst, voff0 + (uint32_t)q * qstep, r, L.kb * 128);
            } else {
                const uint64_t scb = sc_base + (uint64_t)(uint32_t)L.kb * sc_adv;
                const i32x4 sr{(int)(uint32_t)scb, (int)(uint32_t)(scb >> 32) & 0xFFFF, (int)sc_rec & live, 0x00020000};
                dma_lds4(lds0 + SC_BASE + (uint32_t)(L.s * NWAVES * 256 + wave * 256), sc_voff, sr, L.kb * sc_step);
            }
        };
        auto issue_window = [&](const StageLoads& L, auto posc) FP8K_INLINE {
            constexpr int pos = decltype(posc)::value;
            __builtin_amdgcn_sched_barrier(0x0006);
            static_for<NPIECE>([&](auto pc) FP8K_INLINE {
                constexpr int P = decltype(pc)::value;
                if constexpr (P * WIN / NPIECE == pos) issue_piece(L, pc);
            });
            __builtin_amdgcn_sched_barrier(0x0006);
        };
        auto issue_all = [&](const StageLoads& L) FP8K_INLINE { static_for<NPIECE>([&](auto pc) FP8K_INLINE { issue_piece(L, pc); }); };

        auto read_x = [&](int buf, int a, int pr) FP8K_INLINE {
            return *reinterpret_cast<const i32x4*>(smem + buf * BM * 128 + a * 4096 + xa[pr]);
        };
        auto read_w = [&](int buf, int b, int pr) FP8K_INLINE {
            return *reinterpret_cast<const i32x4*>(smem + buf * BN * 128 + b * 4096 + wa[pr]);
        };
        auto read_sa = [&](int buf, int a) FP8K_INLINE {
            return *reinterpret_cast<const float*>(smem + buf * NWAVES * 256 + saa + 128 * a);
        };
        auto read_sb = [&](int buf, int b) FP8K_INLINE {
            return *reinterpret_cast<const float*>(smem + buf * NWAVES * 256 + sb_slot[b]);
        };

        // The tile's K loop, promotion and epilogue for FIV valid 32-row
        // subtiles of this wave (masked layout: the subtiles past the
        // expert's count are neither multiplied nor stored; every other
        // layout: FIV = FI).  The loads and barriers are the same for every
        // FIV, so the waves of a workgroup stay in step.
        if constexpr (MODE == kMasked) {
            auto tile_body = [&](auto fivc) FP8K_INLINE {
                constexpr int FIV = decltype(fivc)::value;
#include "kernels_exact_tile.inc"
            };
            const int fiv = uniform(min(max(rows_valid - wm * TM + 31, 0) / 32, FI));
            static_for<FI + 1>([&](auto fc) FP8K_INLINE {
                if (fiv == decltype(fc)::value) tile_body(fc);
            });
        } else {
            constexpr int FIV = FI;
#include "kernels_exact_tile.inc"
        }
    }
    // the last stages issued were discarded loads; let them retire before the
    // workgroup's LDS is released
    wait_vmcnt<0>();
}

}  // namespace fp8k
