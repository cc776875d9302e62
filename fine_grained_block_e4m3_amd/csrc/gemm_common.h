// gemm_common.h -- pieces shared by the block-scaled GEMM kernels of
// libfp8gemm.so (gfx950): launch parameters, direct-to-LDS loads through
// buffer resources, the LDS chunk swizzle, the tile order and the decoding of
// a tile of the grouped layouts.
#pragma once

#include <type_traits>

#include "device_common.h"

namespace fp8k {

enum GemmMode : int { kDense = 0, kContiguous = 1, kMasked = 2 };

// Operand pointers (passed to the kernel as separate __restrict__ arguments):
//   xq (M, K) codes; masked: (E*max_m, K)
//   sa [K/128][M]; masked: [K/128][E*max_m]
//   wq (N, K); grouped: (E, N, K)
//   sb [ceil(N/128)][K/128]; grouped: (E, N/128, K/128)
//   y  (M, N) BF16 bits; masked: (E*max_m, N)
//   m_indices (contiguous): expert of each row; masked_m (masked): valid rows
struct GemmParams {
    const uint8_t* xq;
    const float* sa;
    const uint8_t* wq;
    const float* sb;
    uint16_t* y;
    uint8_t* yq;                // quantized output (QOUT): E4M3 codes (M, N)
    float* sy;                  // ... and its 1x128 scales [N/128][M]
    const int32_t* m_indices;
    const int32_t* masked_m;
    int64_t M;                  // rows of X (masked: E*max_m)
    int64_t N;                  // output columns (per expert)
    int64_t K;
    int64_t max_m;              // masked only
    int32_t E;
    int64_t m_lo;               // dense/contiguous: tiles cover rows [m_lo, m_lo + m_tiles*BM)
    int64_t n_lo;               // dense: tiles cover columns [n_lo, n_lo + n_tiles*BN) (else 0)
    int32_t m_tiles;            // dense/contiguous: ceil((rows to cover)/BM); masked: ceil(max_m/BM)
    int32_t n_tiles;            // ceil(N/BN)
    int32_t group_m;            // raster group height in tiles
    float* part;                // decode split-K: FP32 partial sums [splits][M][N] (else null)
    int32_t pair_cus;           // contiguous: > 0 when the tiles follow the pair schedule
                                // built on the device (build_pair_sched), with this many
                                // compute units in its full-round rule; 0: rows [m_lo, ...)
};

// Workgroup barrier without a memory fence.  Each wave has already waited on
// its own vector-memory counter for the LDS data it needs; the barrier only
// orders the waves.  (The fence of __syncthreads() would also wait for the
// younger prefetch stages still in flight.)  The memory clobber keeps the
// compiler from moving LDS accesses across it.
__device__ __forceinline__ void lds_barrier() { asm volatile("s_barrier" ::: "memory"); }

// s_waitcnt immediate for "at most n vector-memory operations outstanding"
// (gfx9 encoding: vmcnt[3:0] in bits 3:0 and vmcnt[5:4] in bits 15:14;
// expcnt and lgkmcnt left at their maxima, i.e. not waited on).
template <int n>
__device__ __forceinline__ void wait_vmcnt() {
    static_assert(n >= 0 && n < 64, "vmcnt range");
    __builtin_amdgcn_s_waitcnt((n & 15) | ((n >> 4) << 14) | (7 << 4) | (15 << 8));
}

// Raw buffer resource (V#) over [base, base + bytes), held in SGPRs: loads at
// offsets >= bytes return zeros.  gfx9 dword3: 32-bit data format, raw
// addressing (stride 0).
__device__ __forceinline__ i32x4 make_rsrc(const void* base, uint32_t bytes) {
    const uint64_t b = (uint64_t)base;
    return i32x4{uniform((int)(uint32_t)b), uniform((int)(uint32_t)(b >> 32) & 0xFFFF),
                 uniform((int)bytes), 0x00020000};
}

// A read-only, wave-uniform int32 (here a per-expert count) through the
// scalar cache: an s_load waited on with lgkmcnt, so that it does not wait
// for this wave's outstanding vector loads and stores.
__device__ __forceinline__ int ld_uniform(const int32_t* p, int i) {
    return ((const __attribute__((address_space(4))) int32_t*)(p))[i];
}

// Byte address of an LDS location (the value M0 takes for an LDS DMA).
__device__ __forceinline__ uint32_t lds_addr(const void* p) {
    return (uint32_t)(uintptr_t)(FP8K_LDS const void*)p;
}

// Wave-wide DMAs from a buffer into LDS.  The loads count on this wave's
// vmcnt.  They are issued from asm so that the compiler does not treat them
// as LDS stores that may alias the stage being read (it would wait for every
// DMA in flight).  M0 is restored afterwards.
// One wave-wide 16-byte-per-lane DMA: lane l's bytes land at
// m0 + 1024*Q + 16*l and come from buffer offset voff + 1024*Q + soff.
template <int Q>
__device__ __forceinline__ void dma_lds16_one(uint32_t m0, uint32_t voff, i32x4 rsrc, int soff) {
    int saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dwordx4 %2, %3, %4 offen offset:%5 lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff), "i"(1024 * Q));
}
// One wave-wide DMA of 4 bytes per lane: lane l's dword lands at m0 + 4*l.
__device__ __forceinline__ void dma_lds4(uint32_t m0, uint32_t voff, i32x4 rsrc, int soff) {
    int saved;
    asm volatile("s_mov_b32 %0, m0\n\ts_mov_b32 m0, %1\n\ts_nop 0\n\t"
                 "buffer_load_dword %2, %3, %4 offen lds\n\t"
                 "s_mov_b32 m0, %0"
                 : "=&s"(saved) : "s"(m0), "v"(voff), "s"(rsrc), "s"(soff));
}

// LDS chunk swizzle: chunk c of row r lives in slot c ^ swz(r).  A fragment
// read touches 16 consecutive rows (a 16-aligned run) at one logical chunk;
// with swz(r) = (r mod 8) ^ ((r / 8) mod 2) those reads run at the full LDS
// rate on gfx950 (measured; r mod 8 and (r / 2) mod 8 leave a residual
// conflict).  Depending on r mod 16 only, it keeps every subtile of a wave at
// a fixed offset from the first.
__device__ __forceinline__ int lds_swz(int row) { return (row & 7) ^ ((row >> 3) & 1); }

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

// Number of tiles in the persistent walk.  Dense and contiguous: m_tiles x
// n_tiles.  Masked: each expert's ceil(valid / BM) m-tiles times n_tiles,
// from the device-side counts clamped to [0, max_m] (DeepGEMM page, section
// "分组 GEMM 的两种布局": the masked layout skips the rows past each
// expert's count).
template <int MODE, int BM>
__device__ __forceinline__ int count_tiles(const GemmParams& p, const int32_t* masked_m) {
    if constexpr (MODE == kMasked) {
        int acc = 0;
        for (int e = 0; e < p.E; ++e) {
            int v = ld_uniform(masked_m, e);
            v = v < 0 ? 0 : (v > p.max_m ? (int)p.max_m : v);
            acc += (v + BM - 1) / BM;
        }
        return acc * p.n_tiles;
    } else {
        return p.m_tiles * p.n_tiles;
    }
}

// Where one logical tile of the walk lies.
struct TileCoord {
    int64_t row0;      // first X row of the tile
    int64_t row_end;   // rows [row0, row_end) may be read and written
    int64_t n0;        // first output column
    int expert;        // grouped layouts: whose weights the tile multiplies
};

// Logical tile t -> its rows, columns and expert.  Returns false when the
// tile has nothing to compute (contiguous: a 128-row block of padding only).
//   dense/contiguous: grouped raster order over rows [m_lo, ...);
//   masked: an expert with nmt m-tiles owns logical tiles
//     [base*n_tiles, (base+nmt)*n_tiles), walked m-fastest, so that the
//     m-tiles reading the same W columns run side by side (one XCD, one L2);
//   contiguous: the block's expert is the first index in [0, E) among its
//     rows, in row order (DeepGEMM page, "分组 GEMM 的两种布局": each aligned
//     block belongs to one expert).
template <int MODE, int BM, int BN>
__device__ __forceinline__ bool decode_tile(int t, const GemmParams& p, const int32_t* m_indices,
                                            const int32_t* masked_m, TileCoord& tc) {
    int mt, nt;
    tc.expert = 0;
    if constexpr (MODE == kMasked) {
        const int mt_t = t / p.n_tiles;
        int base = 0, e = 0, valid = 0, nmt = 1;
        for (; e < p.E; ++e) {
            valid = ld_uniform(masked_m, e);
            valid = valid < 0 ? 0 : (valid > p.max_m ? (int)p.max_m : valid);
            nmt = (valid + BM - 1) / BM;
            if (mt_t < base + nmt) break;
            base += nmt;
        }
        tc.expert = e;
        const int local = t - base * p.n_tiles;
        nt = local / nmt;
        mt = local - nt * nmt;
        tc.row0 = (int64_t)e * p.max_m + (int64_t)mt * BM;
        tc.row_end = (int64_t)e * p.max_m + valid;
    } else {
        raster(t, p.m_tiles, p.n_tiles, p.group_m, mt, nt);
        tc.row0 = p.m_lo + (int64_t)mt * BM;
        tc.row_end = p.M;
        if constexpr (MODE == kContiguous) {
            int e = -1;
            for (int r = 0; r < BM && tc.row0 + r < p.M; ++r) {
                const int v = m_indices[tc.row0 + r];
                if (v >= 0 && v < p.E) { e = v; break; }
            }
            if (e < 0) return false;
            tc.expert = e;
        }
    }
    tc.n0 = p.n_lo + (int64_t)nt * BN;
    return true;
}

// Masked layout, largest expert first: logical tile t -> (expert, m tile,
// n tile) with the experts walked in decreasing order of their valid rows
// (ties by index), each expert's tiles m-fastest as in decode_tile.  With one
// workgroup per tile and tile costs that follow the counts, the hardware
// dispatcher then starts the longest tiles first and fills the end of the
// launch with the short ones (longest-processing-time-first list
// scheduling).  Lane l < E takes expert l: its rank and its first m tile of
// the walk come from one pass over the other experts' counts (broadcast from
// their lanes), and the expert whose m-tile range holds t is found by a
// ballot.  E <= 64.  Returns false for t past the walk.
template <int BM, int BN>
__device__ __forceinline__ bool decode_tile_masked_by_count(int t, const GemmParams& p, const int32_t* masked_m,
                                                            TileCoord& tc) {
    const int lane = threadIdx.x & 63;
    int v = lane < p.E ? masked_m[lane] : 0;
    v = v < 0 ? 0 : (v > p.max_m ? (int)p.max_m : v);
    const int nmt = (v + BM - 1) / BM;
    int base = 0;                       // m tiles of the experts walked before this one
    for (int e = 0; e < p.E; ++e) {
        const int ve = __builtin_amdgcn_readlane(v, e);
        const int ne = __builtin_amdgcn_readlane(nmt, e);
        if (ve > v || (ve == v && e < lane)) base += ne;
    }
    const int mt_t = t / p.n_tiles;
    const uint64_t hit = __ballot(lane < p.E && nmt > 0 && mt_t >= base && mt_t < base + nmt);
    if (hit == 0) return false;
    const int e = (int)__builtin_ctzll(hit);
    const int valid = __builtin_amdgcn_readlane(v, e);
    const int nmt_e = __builtin_amdgcn_readlane(nmt, e);
    const int base_e = __builtin_amdgcn_readlane(base, e);
    const int local = t - base_e * p.n_tiles;
    const int nt = local / nmt_e;
    const int mt = local - nt * nmt_e;
    tc.expert = e;
    tc.row0 = (int64_t)e * p.max_m + (int64_t)mt * BM;
    tc.row_end = (int64_t)e * p.max_m + valid;
    tc.n0 = (int64_t)nt * BN;
    return true;
}

// ---------------------------------------------------------------------------
// Contiguous layout, 256-row tiles over pairs of 128-row blocks.  Each
// 128-row aligned block belongs to one expert (DeepGEMM page, "分组 GEMM 的两
// 种布局"), so two consecutive blocks of one expert share their weight tile and
// can run as one 256-row tile.  Within each run of consecutive blocks of one
// expert the blocks pair up in order; a run of odd length leaves its last
// block single.  Three launches share the work, each taking whole rounds of
// its tiles where a last partial round would leave over half of the compute
// units idle and passing the rest on:
//   1. 256x256 tiles over the pairs;
//   2. 128x256 tiles over the blocks left (the singles, then the blocks of
//      the pairs launch 1 passed on);
//   3. 128x64 tiles over the blocks launch 2 passed on.
// Nothing of this is known to the host: every workgroup builds the schedule
// from the row indices into LDS when it starts.
// ---------------------------------------------------------------------------
constexpr int kPairMaxBlocks = 1024;        // 128-row blocks a paired schedule covers (M <= 131072)
constexpr int kPairMaxExperts = 1 << 20;    // experts an entry can name
constexpr int kPairEntries = kPairMaxBlocks + 2;

// Expert of 128-row block b of mt: the first index in [0, E) among its rows,
// in row order (the rule decode_tile follows); -1 for a block with none or
// past the end.
__device__ __forceinline__ int contig_block_expert(const GemmParams& p, const int32_t* m_indices, int b, int mt) {
    if (b >= mt) return -1;
    const int64_t r0 = (int64_t)b * 128, r1 = min(r0 + 128, p.M);
    for (int64_t r = r0; r < r1; ++r) {
        const int v = m_indices[r];
        if (v >= 0 && v < p.E) return v;
    }
    return -1;
}

// Builds the pair schedule into ent (LDS, kPairEntries int32): entries
// b | e << 11 (block b, expert e); the pairs' first blocks, in block order,
// at ent[0 .. P), the singles, in block order, at ent[kPairMaxBlocks - 1],
// ent[kPairMaxBlocks - 2], ...; P and S at ent[kPairMaxBlocks] and
// ent[kPairMaxBlocks + 1].  One wave, all lanes active; the caller checks
// that the blocks fit (mt <= kPairMaxBlocks, so P + S <= kPairMaxBlocks) and
// that E <= kPairMaxExperts.  Lane l takes block 64c + l of chunk c: a block
// starts a run when its expert differs from the one before; it starts a pair
// when it lies an even number of blocks past its run's start and the next
// block has its expert.
__device__ __forceinline__ void build_pair_sched(const GemmParams& p, const int32_t* m_indices, int32_t* ent) {
    const int lane = threadIdx.x & 63;
    const int mt = (int)((p.M + 127) / 128);
    const uint64_t below = (1ull << lane) - 1;
    int np = 0, ns = 0, carry_e = -1, carry_rs = 0;
    for (int c0 = 0; c0 < mt; c0 += 64) {
        const int b = c0 + lane;
        const int e = contig_block_expert(p, m_indices, b, mt);
        const int en = contig_block_expert(p, m_indices, b + 1, mt);
        int ep = __shfl_up(e, 1);
        if (lane == 0) ep = carry_e;
        // run starts at or below this lane (2 << 63 wraps to 0: all lanes)
        const uint64_t starts = __ballot(e >= 0 && e != ep) & ((2ull << lane) - 1);
        const int rs = starts ? c0 + 63 - __clzll((long long)starts) : carry_rs;
        const bool even = ((b - rs) & 1) == 0;
        const bool is_pair = e >= 0 && even && en == e;
        const bool is_single = e >= 0 && even && en != e;
        const uint64_t pm = __ballot(is_pair), sm = __ballot(is_single);
        const int32_t v = b | (e << 11);
        if (is_pair) ent[np + __popcll(pm & below)] = v;
        if (is_single) ent[kPairMaxBlocks - 1 - (ns + __popcll(sm & below))] = v;
        np += __popcll(pm);
        ns += __popcll(sm);
        carry_e = __shfl(e, 63);
        carry_rs = __shfl(rs, 63);
    }
    if (lane == 0) {
        ent[kPairMaxBlocks] = np;
        ent[kPairMaxBlocks + 1] = ns;
    }
}

// Of `units` (pairs or blocks) with nt column tiles each, the ones a launch
// on cus compute units keeps: its whole rounds only, when the last partial
// round would leave over half of the units idle; else all.
__device__ __forceinline__ int units_kept(int units, int nt, int cus) {
    const int tiles = units * nt, full = tiles / cus, last = tiles - full * cus;
    return 2 * last < cus ? full * cus / nt : units;
}

// The share of one launch of the paired schedule (BM x BN: 256x256 launch 1,
// 128x256 launch 2, 128x64 launch 3): its units (pairs or blocks), the first
// of them in the list of blocks left after launch 1 (launch 3), and the
// pairs launch 1 keeps.
struct PairShare {
    int units, first, pm, ns;
};
template <int BM, int BN>
__device__ __forceinline__ PairShare pair_share(const GemmParams& p, const int32_t* ent) {
    static_assert((BM == 256 && BN == 256) || (BM == 128 && (BN == 256 || BN == 64)), "paired launches");
    const int np = uniform(ent[kPairMaxBlocks]), ns = uniform(ent[kPairMaxBlocks + 1]);
    const int nt256 = (int)((p.N + 255) / 256);
    PairShare sh{0, 0, units_kept(np, nt256, p.pair_cus), ns};
    if constexpr (BM == 256) {
        sh.units = sh.pm;
    } else {
        const int left = ns + 2 * (np - sh.pm);
        const int mid = units_kept(left, nt256, p.pair_cus);
        if constexpr (BN == 256) {
            sh.units = mid;
        } else {
            sh.first = mid;
            sh.units = left - mid;
        }
    }
    return sh;
}

// Logical tile t of a paired launch -> its rows, columns and expert.  Block
// u of the list of blocks left: the singles first, then the pairs' blocks.
template <int BM, int BN>
__device__ __forceinline__ void decode_tile_paired(int t, const GemmParams& p, const int32_t* ent,
                                                   const PairShare& sh, TileCoord& tc) {
    int u, nt;
    raster(t, sh.units, p.n_tiles, p.group_m, u, nt);
    int v, b;
    if (BM == 256) {
        v = uniform(ent[u]);
        b = v & 2047;
    } else {
        u += sh.first;
        if (u < sh.ns) {
            v = uniform(ent[kPairMaxBlocks - 1 - u]);
            b = v & 2047;
        } else {
            v = uniform(ent[sh.pm + ((u - sh.ns) >> 1)]);
            b = (v & 2047) + ((u - sh.ns) & 1);
        }
    }
    tc.expert = v >> 11;
    tc.row0 = (int64_t)b * 128;
    tc.row_end = p.M;
    tc.n0 = (int64_t)nt * BN;
}

// Calls f(integral_constant<int, 0>) ... f(integral_constant<int, S-1>) in order.
template <int S, typename F>
__device__ __forceinline__ void static_for(F&& f) {
    if constexpr (S > 0) {
        static_for<S - 1>(f);
        f(std::integral_constant<int, S - 1>{});
    }
}

}  // namespace fp8k
