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
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int64_t K = p.K;
    const int KB = (int)(K / 128);
    const int64_t N = p.N;
    const int h = lane >> 5;            // K half of the block this lane covers
    const int r32 = lane & 31;          // row of a 32-row subtile

    const int total_tiles = count_tiles<MODE, BM>(p, masked_m_);

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
    const uint32_t saa = (uint32_t)(SC_BASE + 4 * (wm * TM + r32));   // + 128*a per subtile
    const bool sa_wave = wave < NSA;
    const uint32_t lds0 = uniform((int)lds_addr(smem));
    const uint32_t ldsw = lds0 + (uint32_t)(wave * 1024);

    // XCD-aware order: workgroup b of a dispatch wave of G lands on XCD b%8;
    // each XCD gets a run of G/8 consecutive logical tiles.
    const int G = gridDim.x;
    const bool remap = (G & 7) == 0;
    const int rounds = (total_tiles + G - 1) / G;

    for (int round = 0; round < rounds; ++round) {
        int t = blockIdx.x;
        if (remap) t = (t & 7) * (G >> 3) + (t >> 3);
        t += round * G;
        if (t >= total_tiles) continue;

        TileCoord tc;
        if (!decode_tile<MODE, BM, BN>(t, p, m_indices_, masked_m_, tc)) continue;
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

        f32x16 acc[FI][FJ];
#pragma unroll
        for (int a = 0; a < FI; ++a)
#pragma unroll
            for (int b = 0; b < FJ; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) acc[a][b][v] = 0.f;

        // ---------------- K loop ----------------
        // Prologue: blocks 0 .. STAGES-2 in full, all in flight together; once
        // block 0 has landed for every wave, window position 0 of block
        // STAGES-1; then the first reads of block 0.  (All waves are done with
        // the previous tile's buffers at the first barrier.  No wait for the
        // vector-memory counter before it: that counter also counts the
        // previous tile's output stores.)
        lds_barrier();
        static_for<STAGES - 1>([&](auto sc) FP8K_INLINE {
            constexpr int b = decltype(sc)::value;
            issue_all(stage_loads(b, b));
        });
        wait_vmcnt<(STAGES - 2) * NPIECE>();
        lds_barrier();
        issue_window(stage_loads(STAGES - 1, STAGES - 1), std::integral_constant<int, 0>{});

        i32x4 rx[FI], rw[FJ];          // raw E4M3 bytes of the current pair of steps
#pragma unroll
        for (int a = 0; a < FI; ++a) rx[a] = read_x(0, a, 0);
#pragma unroll
        for (int b = 0; b < FJ; ++b) rw[b] = read_w(0, b, 0);
        // scales of the current block, and the rescale factors (exponent
        // shifts for power-of-two scales) applied before its first MFMAs
        // (the factor of subtile (a, b) is fa[a] * fb[b], or the shift da[a] + db[b])
        float sa_c[FI], sb_c[FJ];
        float fa[FI], fb[FJ];
        int da[FI], db[FJ];
#pragma unroll
        for (int a = 0; a < FI; ++a) sa_c[a] = read_sa(0, a);
#pragma unroll
        for (int b = 0; b < FJ; ++b) sb_c[b] = read_sb(0, b);
#pragma unroll
        for (int a = 0; a < FI; ++a) {
            fa[a] = 1.f;
            da[a] = 0;
        }
#pragma unroll
        for (int b = 0; b < FJ; ++b) {
            fb[b] = 1.f;
            db[b] = 0;
        }

        // operands of the current MFMA step, widened one step ahead of use
        f16x8 hx[FI], hw[FJ];
#pragma unroll
        for (int a = 0; a < FI; ++a) hx[a] = e4m3x8_to_f16(rx[a][0], rx[a][1]);
#pragma unroll
        for (int b = 0; b < FJ; ++b) hw[b] = e4m3x8_to_f16(rw[b][0], rw[b][1]);

        // Promotion into the next block's units, in the window between a
        // subtile's last MFMA of one block and its first MFMA of the next:
        // half of the subtiles in the block's last step, the other half in
        // the next block's first step, each H = T/2 MFMAs away from the MFMAs
        // on either side, so that the multiplies neither wait for an MFMA
        // result nor hold up the next MFMA (3% on 4096x7168x7168 against
        // rescaling right beside them).
        auto rescale = [&](int a, int b, int v0) FP8K_INLINE {
            const float f = fa[a] * fb[b];
            const int d = da[a] + db[b];
#pragma unroll
            for (int v = v0; v < v0 + 8; ++v) {
                if constexpr (POW2) acc[a][b][v] = __builtin_amdgcn_ldexpf(acc[a][b][v], d);
                else acc[a][b][v] *= f;
            }
        };
        auto block = [&](int kb, auto bufc) FP8K_INLINE {
            constexpr int BUF = decltype(bufc)::value;
            constexpr int NBUF = (BUF + 1) % STAGES;
            // block kb+STAGES-1 (window positions 1 .. into its stage) and
            // kb+STAGES (position 0, after this block's barrier, into BUF)
            const StageLoads L1 = stage_loads(kb + STAGES - 1, (BUF + STAGES - 1) % STAGES);
            const StageLoads L2 = stage_loads(kb + STAGES, BUF);
            const bool last = kb + 1 >= KB;
            float sa_n[FI], sb_n[FJ];
            static_for<NP>([&](auto pc) FP8K_INLINE {
                constexpr int pr = decltype(pc)::value;
                __builtin_amdgcn_sched_barrier(0);
                if constexpr (pr == RB) {
                    // every read of block kb is done (lgkm) and this wave's
                    // loads of block kb+1 have landed; then publish
                    asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
                    wait_vmcnt<(STAGES - 2) * NPIECE>();
                    lds_barrier();
                    __builtin_amdgcn_sched_barrier(0);
                }
                // reads of the next pair: this block, or the next one after the barrier
                constexpr int nbuf = pr + 1 < NP ? BUF : NBUF, npr = (pr + 1) % NP;
                i32x4 nx[FI], nw[FJ];
#pragma unroll
                for (int a = 0; a < FI; ++a) nx[a] = read_x(nbuf, a, npr);
#pragma unroll
                for (int b = 0; b < FJ; ++b) nw[b] = read_w(nbuf, b, npr);
                if constexpr (pr == NP - 1) {
#pragma unroll
                    for (int a = 0; a < FI; ++a) sa_n[a] = read_sa(NBUF, a);
#pragma unroll
                    for (int b = 0; b < FJ; ++b) sb_n[b] = read_sb(NBUF, b);
                }
                if constexpr (pr < RB) issue_window(L1, std::integral_constant<int, pr + 1>{});
                else issue_window(L2, std::integral_constant<int, 0>{});

                static_for<2>([&](auto ec) FP8K_INLINE {
                    constexpr int e = decltype(ec)::value;
                    constexpr bool first = pr == 0 && e == 0, final = pr == NP - 1 && e == 1;
                    // operands of the following step: the second half of this
                    // pair's reads, or the first half of the next pair's
                    f16x8 gx[FI], gw[FJ];
#pragma unroll
                    for (int a = 0; a < FI; ++a)
                        gx[a] = e == 0 ? e4m3x8_to_f16(rx[a][2], rx[a][3]) : e4m3x8_to_f16(nx[a][0], nx[a][1]);
#pragma unroll
                    for (int b = 0; b < FJ; ++b)
                        gw[b] = e == 0 ? e4m3x8_to_f16(rw[b][2], rw[b][3]) : e4m3x8_to_f16(nw[b][0], nw[b][1]);
                    if constexpr (final) {
                        // factors into the next block's units: s_kb / s_kb+1.
                        // A zero scale keeps the current units (factor 1, or
                        // no exponent shift): the block it scales holds zero
                        // codes (the contract of a zero scale), so it adds
                        // nothing in any units.  (Rows past the valid range read zero
                        // scales too; they are never stored.)  After the last
                        // block the factor is 1.  Computed branch-free (the
                        // selects stay inside the MFMA schedule).
#pragma unroll
                        for (int a = 0; a < FI; ++a) {
                            if constexpr (POW2) {
                                int d = e8m0_of(sa_c[a]) - e8m0_of(sa_n[a]);
                                asm volatile("" : "+v"(d));
                                da[a] = (last || sa_n[a] == 0.f) ? 0 : d;
                            } else {
                                float r = sa_c[a] * __builtin_amdgcn_rcpf(sa_n[a]);
                                asm volatile("" : "+v"(r));
                                fa[a] = (last || sa_n[a] == 0.f) ? 1.f : r;
                            }
                        }
#pragma unroll
                        for (int b = 0; b < FJ; ++b) {
                            if constexpr (POW2) {
                                int d = e8m0_of(sb_c[b]) - e8m0_of(sb_n[b]);
                                asm volatile("" : "+v"(d));
                                db[b] = (last || sb_n[b] == 0.f) ? 0 : d;
                            } else {
                                float r = sb_c[b] * __builtin_amdgcn_rcpf(sb_n[b]);
                                asm volatile("" : "+v"(r));
                                fb[b] = (last || sb_n[b] == 0.f) ? 1.f : r;
                            }
                        }
                    }
                    // subtile u < T-H: rescaled in the final step after MFMA u+H;
                    // subtile u >= T-H: in the next block's first step after MFMA
                    // u-(T-H), i.e. H MFMAs away from the MFMAs on either side
                    constexpr int T = FI * FJ, H = T / 2;
                    static_for<T>([&](auto tc) FP8K_INLINE {
                        constexpr int t = decltype(tc)::value, a = t / FJ, b = t % FJ;
                        acc[a][b] = __builtin_amdgcn_mfma_f32_32x32x16_f16(hw[b], hx[a], acc[a][b], 0, 0, 0);
                        if constexpr (final && t >= H) {
                            rescale((t - H) / FJ, (t - H) % FJ, 0);
                            rescale((t - H) / FJ, (t - H) % FJ, 8);
                        }
                        if constexpr (first && t < H) {
                            rescale((t + T - H) / FJ, (t + T - H) % FJ, 0);
                            rescale((t + T - H) / FJ, (t + T - H) % FJ, 8);
                        }
                    });
                    // one MFMA, then its share of the VALU work
                    static_for<FI * FJ>([&](auto) FP8K_INLINE {
                        __builtin_amdgcn_sched_group_barrier(0x008, 1, 0);
                        __builtin_amdgcn_sched_group_barrier(0x002, (first || final) ? 12 : 3, 0);
                    });
#pragma unroll
                    for (int a = 0; a < FI; ++a) hx[a] = gx[a];
#pragma unroll
                    for (int b = 0; b < FJ; ++b) hw[b] = gw[b];
                });
#pragma unroll
                for (int a = 0; a < FI; ++a) rx[a] = nx[a];
#pragma unroll
                for (int b = 0; b < FJ; ++b) rw[b] = nw[b];
            });
            // the next block's scales become current (a zero scale keeps the units)
#pragma unroll
            for (int a = 0; a < FI; ++a) sa_c[a] = (last || sa_n[a] == 0.f) ? sa_c[a] : sa_n[a];
#pragma unroll
            for (int b = 0; b < FJ; ++b) sb_c[b] = (last || sb_n[b] == 0.f) ? sb_c[b] : sb_n[b];
        };
        int kb = 0;
        for (; kb + STAGES <= KB; kb += STAGES)
            static_for<STAGES>([&](auto sc) FP8K_INLINE { block(kb + decltype(sc)::value, sc); });
        static_for<STAGES - 1>([&](auto sc) FP8K_INLINE {
            if (kb + decltype(sc)::value < KB) block(kb + decltype(sc)::value, sc);
        });
        // (the loads issued past the last block were discarded; they retire in
        // order before the next tile's loads, and the kernel's end waits for them)

        // final promotion: out of units of the last block's scale product
#pragma unroll
        for (int a = 0; a < FI; ++a)
#pragma unroll
            for (int b = 0; b < FJ; ++b)
#pragma unroll
                for (int v = 0; v < 16; ++v) {
                    if constexpr (POW2)
                        acc[a][b][v] = __builtin_amdgcn_ldexpf(acc[a][b][v], e8m0_of(sa_c[a]) + e8m0_of(sb_c[b]) - 254);
                    else
                        acc[a][b][v] = (acc[a][b][v] * sa_c[a]) * sb_c[b];
                }

        // ---------------- epilogue ----------------
        // lane l, value v of subtile (a, b): m = wave row + 32a + l%32,
        // n = wave column + 32b + 8*(v/4) + 4*(l/32) + v%4
        if constexpr (QOUT) {
            // E4M3 codes and one scale per 1x128 group along N: the group of
            // row m is this wave's 128 columns, held by lanes l and l^32
            // (DeepGEMM page, section "为什么只做 NT 布局": the activation
            // quantization belongs fused into the kernel that produces them)
#pragma unroll
            for (int a = 0; a < FI; ++a) {
                const int mloc = wm * TM + 32 * a + r32;
                float amax = 0.f;
#pragma unroll
                for (int b = 0; b < FJ; ++b)
#pragma unroll
                    for (int v = 0; v < 16; ++v) amax = fmaxf(amax, fabsf(acc[a][b][v]));
                amax = fmaxf(amax, __shfl_xor(amax, 32));
                if (mloc >= rows_valid) continue;
                const int64_t m = row0 + mloc;
                const float s = group_scale(amax, POW2);
#pragma unroll
                for (int b = 0; b < FJ; ++b)
#pragma unroll
                    for (int q = 0; q < 4; ++q) {
                        const int64_t n = n0 + wn * TN + 32 * b + 8 * q + 4 * h;   // N % 128 == 0
                        if (n < N)
                            *reinterpret_cast<uint32_t*>(p.yq + m * N + n) =
                                cvt_e4m3x4(acc[a][b][4 * q] / s, acc[a][b][4 * q + 1] / s,
                                           acc[a][b][4 * q + 2] / s, acc[a][b][4 * q + 3] / s);
                    }
                const int64_t nw = n0 + wn * TN;
                if (h == 0 && nw < N) p.sy[(nw >> 7) * p.M + m] = s;
            }
            continue;
        }
#pragma unroll
        for (int a = 0; a < FI; ++a) {
            const int mloc = wm * TM + 32 * a + r32;
            const int64_t m = row0 + mloc;
            bool ok = mloc < rows_valid;
            if constexpr (MODE == kContiguous)
                if (ok) ok = m_indices_[m] == expert;
            if (!ok) continue;
            uint16_t* yrow = y_ + m * N;
#pragma unroll
            for (int b = 0; b < FJ; ++b)
#pragma unroll
                for (int q = 0; q < 4; ++q) {
                    const int64_t n = n0 + wn * TN + 32 * b + 8 * q + 4 * h;
                    const uint32_t lo = pack_bf16x2(acc[a][b][4 * q], acc[a][b][4 * q + 1]);
                    const uint32_t hi = pack_bf16x2(acc[a][b][4 * q + 2], acc[a][b][4 * q + 3]);
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
    // the last stages issued were discarded loads; let them retire before the
    // workgroup's LDS is released
    wait_vmcnt<0>();
}

}  // namespace fp8k
