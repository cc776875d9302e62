// kernels_gemm.h -- block-scaled E4M3 NT GEMM for gfx950 (MI355X, CDNA4).
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
//   * FP8_FLAG_UE8M0 (power-of-two scales): the scales are fed to
//     v_mfma_scale_f32_16x16x128_f8f6f4 as E8M0 operands and the whole K
//     loop accumulates inside the matrix core -- no VALU promotion.
//   * Operands reach LDS with global_load_lds_dwordx4 (no VGPR staging).
//     Each tile row is one 128-byte K block; its eight 16-byte chunks are
//     XOR-swizzled by the row index so the fragment reads (16 rows, same
//     chunk) hit distinct banks.  Two LDS stages: the loads of block kb+1
//     fly while block kb is multiplied.
//   * Persistent grid: each workgroup walks tiles with stride gridDim.x
//     (DeepGEMM page, "线程组织": persistent launch with an in-kernel block
//     scheduler; "统一块调度器与 rasterization": grouped raster order so tiles
//     running together share operand rows in L2).
#pragma once

#include "device_common.h"

namespace fp8k {

enum GemmMode : int { kDense = 0, kContiguous = 1, kMasked = 2 };

// How each 128-K block partial is formed.
//   kPathFp8       one FP8 MFMA (16x16x128) per block, VALU promotion by sA*sB
//   kPathFp8Pow2   power-of-two scales as E8M0 operands of the scaled FP8 MFMA,
//                  accumulated over all of K inside the matrix core
//   kPathF16       E4M3 widened to FP16 (exact), four FP16 MFMAs (16x16x32) per
//                  block: exact products, FP32 accumulation; VALU promotion
//   kPathF16Pow2   as kPathF16, promotion by the power-of-two part of each scale
enum GemmPath : int { kPathFp8 = 0, kPathFp8Pow2 = 1, kPathF16 = 2, kPathF16Pow2 = 3 };

struct GemmParams {
    const uint8_t* xq;          // (M, K) codes; masked: (E*max_m, K)
    const float* sa;            // [K/128][M]; masked: [K/128][E*max_m]
    const uint8_t* wq;          // (N, K); grouped: (E, N, K)
    const float* sb;            // [ceil(N/128)][K/128]; grouped: (E, N/128, K/128)
    uint16_t* y;                // (M, N) BF16 bits; masked: (E*max_m, N)
    const int32_t* m_indices;   // contiguous: expert of each row
    const int32_t* masked_m;    // masked: valid rows of each expert
    int64_t M;                  // rows of X (masked: E*max_m)
    int64_t N;                  // output columns (per expert)
    int64_t K;
    int64_t max_m;              // masked only
    int32_t E;
    int32_t m_tiles;            // dense/contiguous: ceil(M/BM); masked: ceil(max_m/BM)
    int32_t n_tiles;            // ceil(N/BN)
    int32_t group_m;            // raster group height in tiles
};

// LDS chunk swizzle: chunk c of row r lives in slot c ^ swz(r).
__device__ __forceinline__ int lds_swz(int row) { return row & 7; }

// Logical tile -> (m tile, n tile) in grouped raster order: group_m m-tiles
// are walked m-fastest for each n tile before the next group of m-tiles.
__device__ __forceinline__ void raster(int t, int m_tiles, int n_tiles, int group_m, int& mt,
                                       int& nt) {
    const int per_group = group_m * n_tiles;
    const int grp = t / per_group;
    const int first = grp * group_m;
    const int gm = min(m_tiles - first, group_m);
    const int r = t - grp * per_group;
    mt = first + r % gm;
    nt = r / gm;
}

template <int BM, int BN, int WAVES_M, int WAVES_N, int MODE, int PATH>
__global__ __launch_bounds__(64 * WAVES_M * WAVES_N, 1) void gemm_kernel(GemmParams p) {
    constexpr int NWAVES = WAVES_M * WAVES_N;
    constexpr int TM = BM / WAVES_M;   // wave tile rows (m)
    constexpr int TN = BN / WAVES_N;   // wave tile columns (n)
    constexpr int FI = TM / 16;        // 16x16 subtiles per wave along m
    constexpr int FJ = TN / 16;        // ... along n
    constexpr int XLOADS = BM / 8 / NWAVES;   // 1 KB direct-to-LDS loads per wave per stage
    constexpr int WLOADS = BN / 8 / NWAVES;
    constexpr int STAGE = (BM + BN) * 128;
    static_assert(TM % 16 == 0 && TN % 16 == 0, "wave tile must be whole 16x16 subtiles");
    static_assert(BM % (8 * NWAVES) == 0 && BN % (8 * NWAVES) == 0, "tile rows per wave");

    __shared__ __attribute__((aligned(1024))) uint8_t smem[2 * STAGE];

    const int lane = threadIdx.x & 63;
    const int wave = uniform(threadIdx.x >> 6);
    const int wm = wave % WAVES_M, wn = wave / WAVES_M;
    const int64_t K = p.K;
    const int KB = (int)(K / 128);
    const int64_t N = p.N;

    // Masked layout: tiles are counted per expert from the device-side counts.
    int total_tiles;
    if constexpr (MODE == kMasked) {
        int acc = 0;
        for (int e = 0; e < p.E; ++e) {
            int v = p.masked_m[e];
            v = v < 0 ? 0 : (v > p.max_m ? (int)p.max_m : v);
            acc += (v + BM - 1) / BM;
        }
        total_tiles = acc * p.n_tiles;
    } else {
        total_tiles = p.m_tiles * p.n_tiles;
    }

    for (int t = blockIdx.x; t < total_tiles; t += gridDim.x) {
        // ---------------- tile decode ----------------
        int mt, nt;
        int64_t row0;       // first X row of the tile
        int64_t row_end;    // rows [row0, row_end) may be read and written
        int expert = 0;
        if constexpr (MODE == kMasked) {
            const int mt_t = t / p.n_tiles;
            nt = t - mt_t * p.n_tiles;
            int base = 0, e = 0, valid = 0;
            for (; e < p.E; ++e) {
                valid = p.masked_m[e];
                valid = valid < 0 ? 0 : (valid > p.max_m ? (int)p.max_m : valid);
                const int nmt = (valid + BM - 1) / BM;
                if (mt_t < base + nmt) break;
                base += nmt;
            }
            expert = e;
            mt = mt_t - base;
            row0 = (int64_t)e * p.max_m + (int64_t)mt * BM;
            row_end = (int64_t)e * p.max_m + valid;
        } else {
            raster(t, p.m_tiles, p.n_tiles, p.group_m, mt, nt);
            row0 = (int64_t)mt * BM;
            row_end = p.M;
            if constexpr (MODE == kContiguous) {
                // expert of this aligned block: its first row naming one in [0, E)
                int e = -1;
                for (int r = 0; r < BM && row0 + r < p.M; ++r) {
                    const int v = p.m_indices[row0 + r];
                    if (v >= 0 && v < p.E) { e = v; break; }
                }
                if (e < 0) continue;   // only padding rows: nothing to compute
                expert = e;
            }
        }
        const int64_t n0 = (int64_t)nt * BN;
        const uint8_t* __restrict__ wq = p.wq;
        const float* __restrict__ sb = p.sb;
        if constexpr (MODE != kDense) {
            wq += (int64_t)expert * N * K;
            sb += (int64_t)expert * (N / 128) * KB;
        }
        const int64_t last_row = row_end - 1;
        const int64_t last_n = N - 1;

        // ---------------- per-lane operand addresses ----------------
        // Direct-to-LDS loads: a wave instruction fills 1 KB = 8 rows; lane l
        // writes slot l%8 of row l/8, which holds logical chunk slot^swz(row).
        const uint8_t* xsrc[XLOADS];
        const uint8_t* wsrc[WLOADS];
        {
            const int rl = lane >> 3, slot = lane & 7;
#pragma unroll
            for (int q = 0; q < XLOADS; ++q) {
                const int r = (wave * XLOADS + q) * 8 + rl;
                int64_t gr = row0 + r;
                gr = gr < last_row ? gr : last_row;
                xsrc[q] = p.xq + gr * K + ((slot ^ lds_swz(r)) << 4);
            }
#pragma unroll
            for (int q = 0; q < WLOADS; ++q) {
                const int r = (wave * WLOADS + q) * 8 + rl;
                int64_t gn = n0 + r;
                gn = gn < last_n ? gn : last_n;
                wsrc[q] = wq + gn * K + ((slot ^ lds_swz(r)) << 4);
            }
        }
        // Activation-scale rows of this lane (one per m subtile).
        int64_t sa_row[FI];
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            int64_t gr = row0 + wm * TM + 16 * i + (lane & 15);
            sa_row[i] = gr < last_row ? gr : last_row;
        }
        // Weight-scale rows (uniform per subtile).
        int sb_row[FJ];
#pragma unroll
        for (int j = 0; j < FJ; ++j) {
            int64_t n = n0 + wn * TN + 16 * j;
            n = n < last_n ? n : last_n;
            sb_row[j] = (int)(n >> 7);
        }

        auto issue_stage = [&](int kb, int buf) {
            uint8_t* base = smem + buf * STAGE;
            const int64_t koff = (int64_t)kb * 128;
#pragma unroll
            for (int q = 0; q < XLOADS; ++q)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(xsrc[q] + koff),
                    (FP8K_LDS void*)(base + (wave * XLOADS + q) * 1024), 16, 0, 0);
#pragma unroll
            for (int q = 0; q < WLOADS; ++q)
                __builtin_amdgcn_global_load_lds(
                    (const void*)(wsrc[q] + koff),
                    (FP8K_LDS void*)(base + BM * 128 + (wave * WLOADS + q) * 1024), 16, 0, 0);
        };

        f32x4 acc[FI][FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i)
#pragma unroll
            for (int j = 0; j < FJ; ++j) acc[i][j] = f32x4{0.f, 0.f, 0.f, 0.f};

        float sa_cur[FI], sa_nxt[FI];
        float sb_cur[FJ], sb_nxt[FJ];
#pragma unroll
        for (int i = 0; i < FI; ++i) sa_cur[i] = p.sa[sa_row[i]];
#pragma unroll
        for (int j = 0; j < FJ; ++j) sb_cur[j] = sb[(int64_t)sb_row[j] * KB];

        issue_stage(0, 0);
        __builtin_amdgcn_s_waitcnt(0);   // vmcnt(0) lgkmcnt(0): stage 0 and scales landed
        __syncthreads();

        const int g = lane >> 4;             // K group of this lane: bytes [32g, 32g+32)
        for (int kb = 0; kb < KB; ++kb) {
            const int buf = kb & 1;
            if (kb + 1 < KB) {
                issue_stage(kb + 1, buf ^ 1);
#pragma unroll
                for (int i = 0; i < FI; ++i) sa_nxt[i] = p.sa[(int64_t)(kb + 1) * p.M + sa_row[i]];
#pragma unroll
                for (int j = 0; j < FJ; ++j) sb_nxt[j] = sb[(int64_t)sb_row[j] * KB + kb + 1];
            }
            const uint8_t* xs = smem + buf * STAGE;
            const uint8_t* ws = xs + BM * 128;

            // X fragments (MFMA B operand): row wm*TM+16i+l%16, bytes [32g, 32g+32)
            i32x8 xf[FI];
#pragma unroll
            for (int i = 0; i < FI; ++i) {
                const int r = wm * TM + 16 * i + (lane & 15);
                const uint8_t* rp = xs + r * 128;
                const i32x4 lo = *reinterpret_cast<const i32x4*>(rp + (((2 * g) ^ lds_swz(r)) << 4));
                const i32x4 hi = *reinterpret_cast<const i32x4*>(rp + (((2 * g + 1) ^ lds_swz(r)) << 4));
                xf[i] = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
            }
            constexpr bool kF16 = PATH == kPathF16 || PATH == kPathF16Pow2;
            constexpr bool kPow2 = PATH == kPathFp8Pow2 || PATH == kPathF16Pow2;
            // FP16 copies of the X fragments (exact widening), four K quarters each
            f16x8 xh[kF16 ? FI : 1][4];
            if constexpr (kF16) {
#pragma unroll
                for (int i = 0; i < FI; ++i)
#pragma unroll
                    for (int q = 0; q < 4; ++q) xh[i][q] = e4m3x8_to_f16(xf[i][2 * q], xf[i][2 * q + 1]);
            }
            float sa_eff[FI];
#pragma unroll
            for (int i = 0; i < FI; ++i) sa_eff[i] = kPow2 ? pow2_part(sa_cur[i]) : sa_cur[i];
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int r = wn * TN + 16 * j + (lane & 15);
                const uint8_t* rp = ws + r * 128;
                const i32x4 lo = *reinterpret_cast<const i32x4*>(rp + (((2 * g) ^ lds_swz(r)) << 4));
                const i32x4 hi = *reinterpret_cast<const i32x4*>(rp + (((2 * g + 1) ^ lds_swz(r)) << 4));
                const i32x8 wf = i32x8{lo[0], lo[1], lo[2], lo[3], hi[0], hi[1], hi[2], hi[3]};
                if constexpr (PATH == kPathFp8Pow2) {
                    const int sw = e8m0_of(sb_cur[j]);
#pragma unroll
                    for (int i = 0; i < FI; ++i)
                        acc[i][j] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                            wf, xf[i], acc[i][j], 0, 0, 0, sw, 0, e8m0_of(sa_cur[i]));
                } else {
                    f32x4 part[FI];
                    if constexpr (kF16) {
                        f16x8 wh[4];
#pragma unroll
                        for (int q = 0; q < 4; ++q) wh[q] = e4m3x8_to_f16(wf[2 * q], wf[2 * q + 1]);
#pragma unroll
                        for (int i = 0; i < FI; ++i) {
                            part[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(
                                wh[0], xh[i][0], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0);
#pragma unroll
                            for (int q = 1; q < 4; ++q)
                                part[i] = __builtin_amdgcn_mfma_f32_16x16x32_f16(wh[q], xh[i][q],
                                                                                 part[i], 0, 0, 0);
                        }
                    } else {
#pragma unroll
                        for (int i = 0; i < FI; ++i)
                            part[i] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                                wf, xf[i], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                    }
                    const float sbj = kPow2 ? pow2_part(sb_cur[j]) : sb_cur[j];
#pragma unroll
                    for (int i = 0; i < FI; ++i) {
                        const float s = sa_eff[i] * sbj;
#pragma unroll
                        for (int r2 = 0; r2 < 4; ++r2) acc[i][j][r2] = fmaf(s, part[i][r2], acc[i][j][r2]);
                    }
                }
            }
            __builtin_amdgcn_s_waitcnt(0);
            __syncthreads();
#pragma unroll
            for (int i = 0; i < FI; ++i) sa_cur[i] = sa_nxt[i];
#pragma unroll
            for (int j = 0; j < FJ; ++j) sb_cur[j] = sb_nxt[j];
        }

        // ---------------- epilogue: BF16 (RNE), predicated stores ----------------
#pragma unroll
        for (int i = 0; i < FI; ++i) {
            const int64_t m = row0 + wm * TM + 16 * i + (lane & 15);
            bool ok = m <= last_row;
            if constexpr (MODE == kContiguous) ok = ok && p.m_indices[m < last_row ? m : last_row] == expert;
            if (!ok) continue;
            uint16_t* yrow = p.y + m * N;
#pragma unroll
            for (int j = 0; j < FJ; ++j) {
                const int64_t n = n0 + wn * TN + 16 * j + 4 * g;
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
}

}  // namespace fp8k
