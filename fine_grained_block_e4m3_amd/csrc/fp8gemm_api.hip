// fp8gemm_api.hip -- host side of libfp8gemm.so: argument validation, kernel
// instance choice and launches for the C ABI declared in include/fp8gemm.h.
//
// Every entry point validates on the host first and enqueues nothing on an
// error; then it launches asynchronously on the caller's stream.  Nothing is
// allocated, freed or synchronized here.
#include <hip/hip_runtime.h>

#include <stdint.h>

#include <atomic>
#include <mutex>

#include "../../include/fp8gemm.h"
#include "kernels_decode.h"
#include "kernels_exact.h"
#include "kernels_gemm.h"
#include "kernels_quant.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;     // rows/cols fit int32 tile math
constexpr int kMaxDevices = 64;
constexpr uint32_t kGemmFlags = FP8_FLAG_UE8M0 | FP8_FLAG_FAST_ACCUM;
// Per-lane operand offsets inside a tile are 32-bit: 256 rows * K < 2^31.
constexpr int64_t kMaxGemmK = (int64_t)1 << 22;

// Per-device compute-unit count, filled once per device.
std::atomic<int> g_cu_count[kMaxDevices];
std::once_flag g_cu_once[kMaxDevices];

fp8_status current_device_cus(int* cus) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return FP8_ERR_NO_DEVICE;
    }
    std::call_once(g_cu_once[dev], [dev]() {
        int n = 0;
        if (hipDeviceGetAttribute(&n, hipDeviceAttributeMultiprocessorCount, dev) != hipSuccess)
            n = 0;
        g_cu_count[dev].store(n);
    });
    const int n = g_cu_count[dev].load();
    if (n <= 0) {
        (void)hipGetLastError();
        return FP8_ERR_NO_DEVICE;
    }
    *cus = n;
    return FP8_OK;
}

bool aligned16(const void* p) { return ((uintptr_t)p & 15u) == 0; }

// Scratch of fp8_gemm_nt_noalloc: the split-K partial sums of the decode GEMM
// in a fixed device array instead of a workspace the caller passes.  Every
// GPU holds its own copy (from when the library is loaded on it until the
// process ends); every call on that GPU shares it.  8 MiB holds the largest
// split the planner picks on a device of up to 341 compute units: splits * N
// stays at or below 96 * CUs columns, and a split decode GEMM has at most 64
// rows of FP32 partial sums (64 * 4 * 96 * 341 bytes < 8 MiB).
constexpr size_t kScratchBytes = (size_t)8 << 20;
static __device__ __align__(256) uint8_t scratch[kScratchBytes];

// Device address of this device's scratch, resolved once per device (the
// array's name is only a host-side stand-in).
void* g_scratch_ptr[kMaxDevices];
hipError_t g_scratch_err[kMaxDevices];
std::once_flag g_scratch_once[kMaxDevices];

fp8_status current_device_scratch(void** ptr) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess || dev < 0 || dev >= kMaxDevices) {
        (void)hipGetLastError();
        return FP8_ERR_NO_DEVICE;
    }
    std::call_once(g_scratch_once[dev], [dev]() {
        void* p = nullptr;
        g_scratch_err[dev] = hipGetSymbolAddress(&p, HIP_SYMBOL(scratch));
        g_scratch_ptr[dev] = g_scratch_err[dev] == hipSuccess ? p : nullptr;
    });
    if (g_scratch_err[dev] != hipSuccess || !g_scratch_ptr[dev]) {
        (void)hipGetLastError();
        return FP8_ERR_NO_DEVICE;
    }
    *ptr = g_scratch_ptr[dev];
    return FP8_OK;
}

fp8_status launch_status() {
    return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// GEMM instances.  Naming: BM x BN workgroup tile, WAVES_M x WAVES_N waves.
// ---------------------------------------------------------------------------
// A persistent launch of `kern` over the tiles of BM x BN: one workgroup per
// compute unit, at most one per tile.  Dense/contiguous: tiles over rows
// [p.m_lo, m_hi) (all rows by default).
// Dense: columns [p.n_lo, n_hi) (all columns by default).  persistent =
// false: one workgroup per possible tile instead.
template <int BM, int BN, int MODE, typename Kernel>
fp8_status launch_tiles(Kernel kern, int threads, fp8k::GemmParams p, int group_m, int cus,
                        hipStream_t stream, int64_t m_hi, bool persistent = true, int64_t n_hi = -1) {
    if (m_hi < 0) m_hi = p.M;
    if (n_hi < 0) n_hi = p.N;
    p.m_tiles = (int)((MODE == fp8k::kMasked ? p.max_m : m_hi - p.m_lo) + BM - 1) / BM;
    p.n_tiles = (int)((n_hi - p.n_lo + BN - 1) / BN);
    p.group_m = group_m;
    int64_t tiles = (int64_t)p.m_tiles * p.n_tiles;
    if (MODE == fp8k::kMasked) tiles *= p.E;   // upper bound; the kernel counts the real ones
    int grid = (int)(tiles < cus || !persistent ? tiles : cus);
    if (grid <= 0) return FP8_OK;
    hipLaunchKernelGGL(kern, dim3(grid), dim3(threads), 0, stream, p.xq, p.sa, p.wq, p.sb, p.y,
                       p.m_indices, p.masked_m, p);
    return launch_status();
}

// The FP8-instruction kernel (FP8_FLAG_FAST_ACCUM and the MX paths).
template <int BM, int BN, int WM, int WN, int MODE, int PATH, int STAGES = 2, int GROUP_M = 4,
          bool QOUT = false>
fp8_status launch_gemm(const fp8k::GemmParams& p, int cus, hipStream_t stream, int64_t m_hi = -1) {
    // masked: one workgroup per possible tile (tile costs follow the counts)
    return launch_tiles<BM, BN, MODE>(fp8k::gemm_kernel<BM, BN, WM, WN, MODE, PATH, STAGES, QOUT>, 64 * WM * WN,
                                      p, GROUP_M, cus, stream, m_hi, MODE != fp8k::kMasked);
}

// The exact-partial kernel (the default path).
template <int BM, int BN, int WM, int WN, int MODE, bool POW2, int STAGES, bool QOUT = false>
fp8_status launch_exact(const fp8k::GemmParams& p, int cus, hipStream_t stream, int64_t m_hi = -1,
                        int64_t n_hi = -1) {
    // masked: the tiles' costs follow the experts' counts (the kernel skips
    // the subtiles past them), so one workgroup per possible tile and the
    // hardware dispatcher balances them
    return launch_tiles<BM, BN, MODE>(fp8k::gemm_exact_kernel<BM, BN, WM, WN, MODE, POW2, STAGES, QOUT>,
                                      64 * WM * WN, p, 4, cus, stream, m_hi, MODE != fp8k::kMasked, n_hi);
}

// ---------------------------------------------------------------------------
// Instance choice.  Pure integer arithmetic on the shape and the compute-unit
// count, so that fp8_gemm_plan can report it and tests can check it on the
// host; the launches below follow the plan.
// ---------------------------------------------------------------------------
int64_t cdiv(int64_t a, int64_t b) { return (a + b - 1) / b; }

enum Inst : int {
    // FP8-instruction kernel (FP8_FLAG_FAST_ACCUM, MX paths)
    kFastDecode, kFastDecodeKx, kFast64x96, kFast256x224, kFast256x256, kFast256x128, kFast128x128,
    kFast128x256, kFast128x64,
    // exact-partial kernel (default)
    kExact64x96, kExact256x256, kExact256x192, kExact128x256, kExact128x128, kExact128x64, kExactQ256x256,
    kExactQ128x256,
    kExactDecode, kExactDecodeX,
};

// Exact decode kernel: 32 W rows per wave, kExactDecodeNW waves per
// workgroup, a W ring of kExactDecodeNS K blocks per wave, X in chunks of
// kExactDecodeKBC K blocks.
constexpr int kExactDecodeNW = 3, kExactDecodeNS = 5, kExactDecodeKBC = 4;
// X-resident variant: at most kbmax K blocks per workgroup (its X range, sA
// and the W rings fit in LDS), a W ring of kExactDecodeXNS blocks per wave.
constexpr int kExactDecodeXNS = 4;
constexpr int exact_decode_kbmax(int64_t M) { return M <= 32 ? 24 : 12; }

struct InstInfo { int bm, bn, waves, kernel, exact; };
InstInfo inst_info(Inst i) {
    switch (i) {
        case kFastDecode: return {32, 96, 6, 1, 0};
        case kFastDecodeKx: return {48, 96, 8, 2, 0};
        case kFast64x96: return {64, 96, 4, 0, 0};
        case kFast256x224: return {256, 224, 8, 0, 0};
        case kFast256x256: return {256, 256, 8, 0, 0};
        case kFast256x128: return {256, 128, 8, 0, 0};
        case kFast128x128: return {128, 128, 4, 0, 0};
        case kFast128x256: return {128, 256, 8, 0, 0};
        case kFast128x64: return {128, 64, 8, 0, 0};
        case kExact64x96: return {64, 96, 6, 0, 1};
        case kExact256x256: return {256, 256, 8, 0, 1};
        case kExact256x192: return {256, 192, 8, 0, 1};
        case kExact128x256: return {128, 256, 8, 0, 1};
        case kExact128x128: return {128, 128, 4, 0, 1};
        case kExact128x64: return {128, 64, 8, 0, 1};
        case kExactQ256x256: return {256, 256, 8, 0, 1};
        case kExactQ128x256: return {128, 256, 4, 0, 1};
        case kExactDecode: return {64, 32 * kExactDecodeNW, kExactDecodeNW, 3, 1};
        case kExactDecodeX: return {64, 32 * kExactDecodeNW, kExactDecodeNW, 4, 1};
    }
    return {0, 0, 0, 0, 0};
}

// Decode split-K: workgroups along K per column tile of a decode kernel
// (tile_n columns, K in chunks of kbc blocks), when the column tiles are
// fewer than the compute units and the caller's workspace holds the partial
// sums.
constexpr int kDecodeTileN = 96;
size_t decode_ws_bytes(int64_t splits, int64_t M, int64_t N) { return (size_t)(splits * M * N) * sizeof(float); }
int64_t decode_splits(int64_t M, int64_t N, int64_t K, int cus, size_t ws_bytes, int tile_n, int kbc) {
    const int64_t tiles = cdiv(N, tile_n);
    const int64_t nct = cdiv(K / 128, kbc);
    int64_t splits = tiles < cus ? cus / tiles : 1;
    if (splits > nct) splits = nct;
    if (splits > 8) splits = 8;
    if (splits < 1) splits = 1;
    if (splits > 1 && decode_ws_bytes(splits, M, N) > ws_bytes) splits = 1;
    return splits;
}

struct Plan {
    Inst main;
    int64_t main_rows;      // contiguous: the main launch covers rows [0, main_rows)
    Inst tail;              // contiguous: the launch over [main_rows, M), if main_rows < M;
                            // dense: the launch over columns [main_cols, N), if main_cols > 0
    int64_t k_splits;       // decode kernel
    int64_t main_cols = 0;  // dense, > 0: the main launch covers columns [0, main_cols)
    bool paired = false;    // contiguous: main over pairs of 128-row blocks, then mid
    Inst mid = kFast128x128; // and tail over the blocks left (gemm_common.h: pair schedule)
};

// The FP8-instruction paths.  Compute-bound shapes use 8 waves (2 per SIMD)
// so that one wave's promotion FMAs run while the other wave's MFMAs occupy
// the matrix core.
Plan plan_fast(int mode, int64_t M, int64_t N, int64_t K, bool mx, bool qout, int cus, size_t ws_bytes,
               bool pair) {
    Plan pl{kFast128x128, M, kFast128x128, 1};
    if (mode == fp8k::kDense) {
        if (qout) {
            // quantized output: 128-column output groups need a tile width of
            // 128 or 256 with 64-column waves
            if (cdiv(M, 256) * cdiv(N, 256) >= cus) pl.main = kFast256x256;
            else if (cdiv(M, 256) * cdiv(N, 128) >= 2 * cus) pl.main = kFast256x128;
            else pl.main = kFast128x128;
            return pl;
        }
        if (M <= 64) {
            // M <= 32: the decode kernel (96 columns per workgroup, one wave
            // per 16 W rows).  Above 32 rows each of its waves re-reads an X
            // block larger than its W block from LDS; 33..48 rows with
            // K <= 1664 take the X-resident decode kernel (waves splitting K),
            // and the rest the 64x96 tile of the main kernel.  Kernel trace,
            // N 24576, K 1536: M 16 7.3 vs 10.3 us (64x96), M 32 8.8 vs 10.3,
            // M 48 9.6 (X-resident) vs 10.4, M 64 10.7 (X-resident) and 12.2
            // (decode) vs 10.0-10.4.  A 32-column decode workgroup (more of
            // them, several per CU) measured slower on every shape tried.
            if (!mx && M <= 32) {
                pl.main = kFastDecode;
                pl.k_splits = decode_splits(M, N, K, cus, ws_bytes, kDecodeTileN, 4);
            } else if (!mx && M <= 48 && K <= fp8k::kDecodeKxMaxK) {
                pl.main = kFastDecodeKx;
            } else {
                pl.main = kFast64x96;
            }
            return pl;
        }
        const int64_t huge = cdiv(M, 256) * cdiv(N, 256);
        if (huge >= cus) {
            // 256x224 when it takes fewer waves' worth of tile area (e.g.
            // N = 7168: 32 tiles of 224 per row fill two whole waves where
            // 28 tiles of 256 leave the second one a quarter empty; the
            // DeepGEMM page, section "非对齐块大小", makes the same trade
            // with 112-column blocks)
            const int64_t t224 = cdiv(M, 256) * cdiv(N, 224);
            const int64_t cost256 = cdiv(huge, cus) * 256;
            const int64_t cost224 = cdiv(t224, cus) * 224;
            pl.main = cost224 < cost256 ? kFast256x224 : kFast256x256;
        } else if (cdiv(M, 256) * cdiv(N, 128) >= 2 * cus) {
            pl.main = kFast256x128;
        } else {
            pl.main = kFast128x128;
        }
    } else if (mode == fp8k::kContiguous && pair && cdiv(M, 128) <= fp8k::kPairMaxBlocks &&
               cdiv(M, 256) * cdiv(N, 256) >= cus) {
        // the pair schedule, as on the exact path
        pl.main = kFast256x256;
        pl.mid = kFast128x256;
        pl.tail = kFast128x64;
        pl.paired = true;
    } else if (mode == fp8k::kContiguous) {
        // The M tile must equal the layout alignment (128): one expert per
        // tile.  When the last round of 128x256 tiles would leave over half of
        // the CUs idle, the full rounds' 128-row blocks run as one launch and
        // the remaining blocks as a second one with 128x64 tiles (8 waves of
        // 32x32), four times as many (8 experts x 8192 tokens, N 4096: 1088
        // tiles = 4.25 rounds -> 4 full rounds + 256 tiles of 128x64;
        // measured 343 -> 327 us).
        pl.main = kFast128x256;
        const int64_t mt = cdiv(M, 128), nt = cdiv(N, 256);
        const int64_t full = mt * nt / cus, last = mt * nt - full * cus;
        const int64_t m_main = full * cus / nt;   // 128-row blocks of the full rounds
        if (full >= 1 && 2 * last < cus && m_main < mt) {
            pl.main_rows = m_main * 128;
            pl.tail = kFast128x64;
        }
    } else {
        // Masked: 256-row tiles of 2x4 waves, one workgroup per possible tile,
        // the waves skipping the 16-row subtiles past the expert's count and
        // the tiles walked largest expert first (as on the default path);
        // before: persistent 128x256 tiles (128-row tiles padded each
        // expert's rows less than 256-row ones without the skip).
        pl.main = kFast256x256;
    }
    return pl;
}

// The exact-partial path (FP16 matrix instruction on E4M3 operands widened
// exactly).  Waves hold 64x128 (or 64x64) of 32x32 subtiles.
// Dense, 256-row tiles: the columns [0, c) in 256x256 tiles and the rest in
// 256x192 tiles, as two launches, when that takes fewer rounds' worth of tile
// width than 256x256 tiles throughout (the round time of a launch taken as
// proportional to its tile width).  4096 x 7168 on 256 CUs: 448 tiles of 256
// are 1.75 rounds, so the second round leaves a quarter of the CUs idle;
// columns [0, 4096) as 256 tiles of 256 and [4096, 7168) as 256 tiles of 192
// are one round each (the DeepGEMM page, section "非对齐块大小", makes the same
// trade with 112-column blocks).  Returns c, or 0 to keep one launch.
int64_t exact_split_cols(int64_t M, int64_t N, int cus) {
    const int64_t mt = cdiv(M, 256), nt = cdiv(N, 256);
    int64_t best = cdiv(mt * nt, cus) * 256, cols = 0;
    for (int64_t j = 1; j < nt; ++j) {
        const int64_t w = cdiv(mt * j, cus) * 256 + cdiv(mt * cdiv(N - 256 * j, 192), cus) * 192;
        if (w < best || (cols > 0 && w == best)) {   // ties: the most columns in 256x256 tiles
            best = w;
            cols = 256 * j;
        }
    }
    return cols;
}

Plan plan_exact(int mode, int64_t M, int64_t N, int64_t K, bool qout, int cus, size_t ws_bytes, bool pair) {
    Plan pl{kExact128x128, M, kExact128x128, 1};
    if (mode == fp8k::kDense) {
        if (qout) {
            // a 1x128 output group per wave: 128-column waves
            pl.main = cdiv(M, 256) * cdiv(N, 256) >= cus ? kExactQ256x256 : kExactQ128x256;
        } else if (M <= 64) {
            // decode-sized M.  With few column tiles (and a workspace) K is
            // split over workgroups: the exact decode kernel with X resident
            // when each range holds at most kbmax blocks, else with X in
            // chunks.  Unsplit, M <= 32 takes the decode kernel, M > 32 the
            // 64x96 tile of the main kernel (kernel trace, N 24576, K 1536:
            // M 64 20.0 vs 15.4 us, M 48 19.8 vs 15.1, M 32 13.8 vs 14.6,
            // M 16 14.3 vs 14.4; N 4096, K 7168: M 16 16.9 us split vs 40
            // unsplit).
            const int64_t sx = decode_splits(M, N, K, cus, ws_bytes, 32 * kExactDecodeNW, 1);
            const bool fits = cdiv(K / 128, sx) <= exact_decode_kbmax(M);
            if (sx == 1 && M <= 32 && cdiv(N, 32 * kExactDecodeNW) >= cus) {
                // a whole round of column tiles, unsplit: X in chunks beats X
                // resident (N 24576: M 1-32, K 1536 12.4-12.9 vs 13.1-13.6 us,
                // M 32, K 3072 20.2 vs 21.4; with fewer tiles the resident X
                // wins: 16x7168x2048 11.8 vs 12.7)
                pl.main = kExactDecode;
            } else if (fits && (sx > 1 || M <= 32)) {
                pl.main = kExactDecodeX;
                pl.k_splits = sx;
            } else if (sx == 1 && M > 32) {
                pl.main = kExact64x96;
            } else {
                pl.main = kExactDecode;
                pl.k_splits = decode_splits(M, N, K, cus, ws_bytes, 32 * kExactDecodeNW, kExactDecodeKBC);
            }
        } else if (cdiv(M, 256) * cdiv(N, 256) >= cus) {
            pl.main = kExact256x256;
            pl.main_cols = exact_split_cols(M, N, cus);
            if (pl.main_cols > 0) pl.tail = kExact256x192;
        } else if (cdiv(M, 128) * cdiv(N, 256) >= cus) {
            pl.main = kExact128x256;
        } else {
            pl.main = kExact128x128;
        }
    } else if (mode == fp8k::kContiguous && pair && cdiv(M, 128) <= fp8k::kPairMaxBlocks &&
               cdiv(M, 256) * cdiv(N, 256) >= cus) {
        // 256-row tiles over pairs of one expert's 128-row blocks, then
        // 128x256 and 128x64 tiles over the blocks left, the split found on
        // the device (gemm_common.h).  8 experts x 8192 tokens, N 4096: 32
        // pairs + 4 single blocks = 2 rounds of 256x256 tiles and one of
        // 128x64 tiles, against 4 rounds of 128x256 tiles and one of 128x64.
        pl.main = kExact256x256;
        pl.mid = kExact128x256;
        pl.tail = kExact128x64;
        pl.paired = true;
    } else if (mode == fp8k::kContiguous) {
        // 128-row tiles (the layout alignment); the blocks past the last full
        // round of 128x256 tiles run as 128x64 tiles of 8 waves (32x32 each)
        // when that round would leave over half of the CUs idle (8 experts x
        // 8192 tokens, N 4096: the tail launch takes 51 us against 83 us for
        // 128x128 tiles of 4 waves, kernel trace)
        pl.main = kExact128x256;
        const int64_t mt = cdiv(M, 128), nt = cdiv(N, 256);
        const int64_t full = mt * nt / cus, last = mt * nt - full * cus;
        const int64_t m_main = full * cus / nt;
        if (full >= 1 && 2 * last < cus && m_main < mt) {
            pl.main_rows = m_main * 128;
            pl.tail = kExact128x64;
        }
    } else {
        // masked: 256-row tiles of 2x4 waves (128x64 each), one workgroup per
        // possible tile; the waves skip the 32-row subtiles past the expert's
        // count (16 experts x 256 rows, N 7168, K 2048: 94 us against 105 us
        // for persistent 128x256 tiles, 110 us for 256x256 tiles with the
        // other wave order, 116 us without the skip; one box)
        pl.main = kExact256x256;
    }
    return pl;
}

// pair: the contiguous pair schedule may be used (E <= kPairMaxExperts).
Plan make_plan(int mode, int64_t M, int64_t N, int64_t K, uint32_t flags, bool mx, bool qout, int cus,
               size_t ws_bytes, bool pair = true) {
    return (mx || (flags & FP8_FLAG_FAST_ACCUM)) ? plan_fast(mode, M, N, K, mx, qout, cus, ws_bytes, pair)
                                                 : plan_exact(mode, M, N, K, qout, cus, ws_bytes, pair);
}

// ---------------------------------------------------------------------------
// Launches.
// ---------------------------------------------------------------------------
// Decode-sized dense GEMM (M <= 32): one workgroup per 16*NW output columns
// and all M rows, one wave per 16 columns; MSUB = ceil(M/16) row subtiles.
// With splits > 1 the K chunks are split over that many workgroups per tile:
// they write FP32 partial sums to the caller's workspace and a second kernel
// adds them in split order and rounds to BF16.
template <int NW, int NS, bool POW2>
fp8_status launch_decode(const fp8k::GemmParams& p0, int64_t splits, void* ws, hipStream_t stream) {
    static_assert(16 * NW == kDecodeTileN, "decode tile width");
    fp8k::GemmParams p = p0;
    const int64_t tiles = cdiv(p.N, 16 * NW);
    if (tiles <= 0) return FP8_OK;
    if (splits <= 1) ws = nullptr;
    p.part = static_cast<float*>(ws);
    const dim3 grid((unsigned)tiles, (unsigned)(ws ? splits : 1)), block(64 * NW);
    switch ((p.M + 15) / 16) {
        case 1: hipLaunchKernelGGL((fp8k::decode_kernel<1, NW, NS, POW2>), grid, block, 0, stream,
                                   p.xq, p.sa, p.wq, p.sb, p.y, p); break;
        case 2: hipLaunchKernelGGL((fp8k::decode_kernel<2, NW, NS, POW2>), grid, block, 0, stream,
                                   p.xq, p.sa, p.wq, p.sb, p.y, p); break;
        default: return FP8_ERR_UNSUPPORTED;
    }
    fp8_status st = launch_status();
    if (ws && st == FP8_OK) {
        const int64_t mn = p.M * p.N;
        hipLaunchKernelGGL(fp8k::decode_split_reduce, dim3((unsigned)cdiv(mn, 256)), dim3(256), 0, stream,
                           static_cast<const float*>(ws), (int)splits, mn, p.y);
        st = launch_status();
    }
    return st;
}

// Decode-sized dense GEMM with 32 < M <= 48 and K <= kDecodeKxMaxK: X resident
// in LDS, waves splitting K.
template <bool POW2>
fp8_status launch_decode_kx(const fp8k::GemmParams& p, hipStream_t stream) {
    const int64_t tiles = cdiv(p.N, 96);
    if (tiles <= 0) return FP8_OK;
    hipLaunchKernelGGL((fp8k::decode_kx_kernel<3, POW2>), dim3((unsigned)tiles), dim3(512), 0, stream,
                       p.xq, p.sa, p.wq, p.sb, p.y, p);
    return launch_status();
}

// One launch of instance `i` (m_hi: dense/contiguous rows [p.m_lo, m_hi)).
template <int MODE, int PATH>
fp8_status launch_fast(Inst i, const fp8k::GemmParams& p, int64_t splits, void* ws, int cus, hipStream_t stream,
                       int64_t m_hi, bool qout) {
    constexpr bool kPow2 = PATH == fp8k::kPathFp8Pow2;
    constexpr bool kBlock = PATH == fp8k::kPathFp8 || PATH == fp8k::kPathFp8Pow2;
    if constexpr (MODE == fp8k::kDense) {
        if constexpr (kBlock) {
            if (qout) {
                switch (i) {
                    case kFast256x256: return launch_gemm<256, 256, 2, 4, MODE, PATH, 2, 4, true>(p, cus, stream);
                    case kFast256x128: return launch_gemm<256, 128, 4, 2, MODE, PATH, 3, 4, true>(p, cus, stream);
                    case kFast128x128: return launch_gemm<128, 128, 2, 2, MODE, PATH, 4, 4, true>(p, cus, stream);
                    default: return FP8_ERR_UNSUPPORTED;
                }
            }
            if (i == kFastDecode) return launch_decode<6, 5, kPow2>(p, splits, ws, stream);
            if (i == kFastDecodeKx) return launch_decode_kx<kPow2>(p, stream);
        }
        switch (i) {
            case kFast64x96: return launch_gemm<64, 96, 2, 2, MODE, PATH, 3>(p, cus, stream);
            case kFast256x224: return launch_gemm<256, 224, 4, 2, MODE, PATH>(p, cus, stream);
            case kFast256x256: return launch_gemm<256, 256, 2, 4, MODE, PATH>(p, cus, stream);
            case kFast256x128: return launch_gemm<256, 128, 4, 2, MODE, PATH, 3>(p, cus, stream);
            case kFast128x128: return launch_gemm<128, 128, 2, 2, MODE, PATH, 4>(p, cus, stream);
            default: return FP8_ERR_UNSUPPORTED;
        }
    } else if constexpr (kBlock) {
        switch (i) {
            case kFast128x256:
                if constexpr (MODE == fp8k::kContiguous) return launch_gemm<128, 256, 2, 4, MODE, PATH, 3>(p, cus, stream, m_hi);
                else return FP8_ERR_UNSUPPORTED;
            case kFast256x256: return launch_gemm<256, 256, 2, 4, MODE, PATH, 2>(p, cus, stream, m_hi);
            case kFast128x64:
                if constexpr (MODE == fp8k::kContiguous) return launch_gemm<128, 64, 4, 2, MODE, PATH, 4>(p, cus, stream, m_hi);
                else return FP8_ERR_UNSUPPORTED;
            default: return FP8_ERR_UNSUPPORTED;
        }
    } else {
        return FP8_ERR_UNSUPPORTED;
    }
}

// Exact decode GEMM (M <= 64): one workgroup per 32*NW output columns and all
// M rows; MSUB = ceil(M/32) row subtiles.  With splits > 1 the K chunks are
// split over that many workgroups per tile (FP32 partial sums in the
// caller's workspace, added in split order by a second kernel).
template <int NW, int NS, int KBC>
fp8_status launch_decode_exact(const fp8k::GemmParams& p0, int64_t splits, void* ws, hipStream_t stream) {
    fp8k::GemmParams p = p0;
    const int64_t tiles = cdiv(p.N, 32 * NW);
    if (tiles <= 0) return FP8_OK;
    if (splits <= 1) ws = nullptr;
    p.part = static_cast<float*>(ws);
    const dim3 grid((unsigned)tiles, (unsigned)(ws ? splits : 1)), block(64 * NW);
    switch ((p.M + 31) / 32) {
        case 1: hipLaunchKernelGGL((fp8k::decode_exact_kernel<1, NW, NS, KBC>), grid, block, 0, stream,
                                   p.xq, p.sa, p.wq, p.sb, p.y, p); break;
        case 2: hipLaunchKernelGGL((fp8k::decode_exact_kernel<2, NW, NS, KBC>), grid, block, 0, stream,
                                   p.xq, p.sa, p.wq, p.sb, p.y, p); break;
        default: return FP8_ERR_UNSUPPORTED;
    }
    fp8_status st = launch_status();
    if (ws && st == FP8_OK) {
        const int64_t mn = p.M * p.N;
        hipLaunchKernelGGL(fp8k::decode_split_reduce, dim3((unsigned)cdiv(mn, 256)), dim3(256), 0, stream,
                           static_cast<const float*>(ws), (int)splits, mn, p.y);
        st = launch_status();
    }
    return st;
}

// The X-resident variant: K blocks [s*KB/S, (s+1)*KB/S) per workgroup (at
// most exact_decode_kbmax(M) of them, which the plan ensures).
template <int NW, int NS>
fp8_status launch_decode_exact_x(const fp8k::GemmParams& p0, int64_t splits, void* ws, hipStream_t stream) {
    fp8k::GemmParams p = p0;
    const int64_t tiles = cdiv(p.N, 32 * NW);
    if (tiles <= 0) return FP8_OK;
    if (splits <= 1) ws = nullptr;
    const int64_t s = ws ? splits : 1;
    if (s > p.K / 128 || cdiv(p.K / 128, s) > exact_decode_kbmax(p.M)) return FP8_ERR_UNSUPPORTED;
    p.part = static_cast<float*>(ws);
    const dim3 grid((unsigned)tiles, (unsigned)s), block(64 * NW);
    switch ((p.M + 31) / 32) {
        case 1: hipLaunchKernelGGL((fp8k::decode_exact_x_kernel<1, NW, NS, 24>), grid, block, 0, stream,
                                   p.xq, p.sa, p.wq, p.sb, p.y, p); break;
        case 2: hipLaunchKernelGGL((fp8k::decode_exact_x_kernel<2, NW, NS, 12>), grid, block, 0, stream,
                                   p.xq, p.sa, p.wq, p.sb, p.y, p); break;
        default: return FP8_ERR_UNSUPPORTED;
    }
    fp8_status st = launch_status();
    if (ws && st == FP8_OK) {
        const int64_t mn = p.M * p.N;
        hipLaunchKernelGGL(fp8k::decode_split_reduce, dim3((unsigned)cdiv(mn, 256)), dim3(256), 0, stream,
                           static_cast<const float*>(ws), (int)splits, mn, p.y);
        st = launch_status();
    }
    return st;
}

template <int MODE, bool POW2>
fp8_status launch_exact_inst(Inst i, const fp8k::GemmParams& p, int64_t splits, void* ws, int cus,
                             hipStream_t stream, int64_t m_hi, int64_t n_hi = -1) {
    if constexpr (MODE == fp8k::kDense) {
        switch (i) {
            case kExact64x96: return launch_exact<64, 96, 2, 3, MODE, POW2, 3>(p, cus, stream);
            case kExact256x256: return launch_exact<256, 256, 4, 2, MODE, POW2, 2>(p, cus, stream, -1, n_hi);
            case kExact256x192: return launch_exact<256, 192, 4, 2, MODE, POW2, 2>(p, cus, stream);
            case kExact128x256: return launch_exact<128, 256, 2, 4, MODE, POW2, 3>(p, cus, stream);
            case kExact128x128: return launch_exact<128, 128, 2, 2, MODE, POW2, 4>(p, cus, stream);
            case kExactQ256x256: return launch_exact<256, 256, 4, 2, MODE, POW2, 2, true>(p, cus, stream);
            case kExactQ128x256: return launch_exact<128, 256, 2, 2, MODE, POW2, 3, true>(p, cus, stream);
            case kExactDecode:
                return launch_decode_exact<kExactDecodeNW, kExactDecodeNS, kExactDecodeKBC>(p, splits, ws, stream);
            case kExactDecodeX: return launch_decode_exact_x<kExactDecodeNW, kExactDecodeXNS>(p, splits, ws, stream);
            default: return FP8_ERR_UNSUPPORTED;
        }
    } else {
        switch (i) {
            case kExact128x256:
                if constexpr (MODE == fp8k::kContiguous) return launch_exact<128, 256, 2, 4, MODE, POW2, 3>(p, cus, stream, m_hi);
                else return FP8_ERR_UNSUPPORTED;
            case kExact256x256:
                if constexpr (MODE == fp8k::kMasked) return launch_exact<256, 256, 2, 4, MODE, POW2, 2>(p, cus, stream, m_hi);
                else return launch_exact<256, 256, 4, 2, MODE, POW2, 2>(p, cus, stream, m_hi);
            case kExact128x64:
                if constexpr (MODE == fp8k::kContiguous) return launch_exact<128, 64, 4, 2, MODE, POW2, 4>(p, cus, stream, m_hi);
                else return FP8_ERR_UNSUPPORTED;
            default: return FP8_ERR_UNSUPPORTED;
        }
    }
}

// Runs a plan: the main launch, then (contiguous) the tail launch.
template <int MODE, int PATH>
fp8_status run_plan(const Plan& pl, bool exact, const fp8k::GemmParams& p, void* ws, int cus,
                    hipStream_t stream, bool qout) {
    constexpr bool kPow2 = PATH == fp8k::kPathFp8Pow2;
    auto one = [&](Inst i, const fp8k::GemmParams& q, int64_t m_hi) {
        return exact ? launch_exact_inst<MODE, kPow2>(i, q, pl.k_splits, ws, cus, stream, m_hi)
                     : launch_fast<MODE, PATH>(i, q, pl.k_splits, ws, cus, stream, m_hi, qout);
    };
    if (MODE == fp8k::kDense && exact && pl.main_cols > 0 && pl.main_cols < p.N) {
        // columns [0, main_cols), then [main_cols, N) with the narrower tile
        fp8_status st = launch_exact_inst<MODE, kPow2>(pl.main, p, 1, ws, cus, stream, -1, pl.main_cols);
        if (st != FP8_OK) return st;
        fp8k::GemmParams t = p;
        t.n_lo = pl.main_cols;
        return one(pl.tail, t, -1);
    }
    if (MODE == fp8k::kContiguous && pl.paired) {
        // the three launches of the pair schedule, each finding its share on
        // the device
        fp8k::GemmParams q = p;
        q.pair_cus = cus;
        for (Inst i : {pl.main, pl.mid, pl.tail}) {
            const fp8_status st = one(i, q, -1);
            if (st != FP8_OK) return st;
        }
        return FP8_OK;
    }
    if (MODE == fp8k::kContiguous && pl.main_rows < p.M) {
        fp8_status st = one(pl.main, p, pl.main_rows);
        if (st != FP8_OK) return st;
        fp8k::GemmParams t = p;
        t.m_lo = pl.main_rows;
        return one(pl.tail, t, -1);
    }
    return one(pl.main, p, -1);
}

// Block-scaled GEMM call of layout MODE: plan, then launch.
template <int MODE>
fp8_status run_gemm(const fp8k::GemmParams& p, uint32_t flags, void* ws, size_t ws_bytes, hipStream_t stream,
                    bool qout = false) {
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    const Plan pl = make_plan(MODE, p.M, p.N, p.K, flags, false, qout, cus, ws_bytes, p.E <= fp8k::kPairMaxExperts);
    const bool exact = !(flags & FP8_FLAG_FAST_ACCUM);
    return (flags & FP8_FLAG_UE8M0) ? run_plan<MODE, fp8k::kPathFp8Pow2>(pl, exact, p, ws, cus, stream, qout)
                                    : run_plan<MODE, fp8k::kPathFp8>(pl, exact, p, ws, cus, stream, qout);
}

bool dims_ok(int64_t a) { return a >= 0 && a < kMaxDim; }

// MXFP8 / MXFP4 weights: the dense FP8-instruction instances with the MX path
// (scales as per-lane E8M0 operands, no promotion).
template <int PATH>
fp8_status run_gemm_mx(const fp8k::GemmParams& p, hipStream_t stream) {
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    const Plan pl = make_plan(fp8k::kDense, p.M, p.N, p.K, 0, true, false, cus, 0);
    return launch_fast<fp8k::kDense, PATH>(pl.main, p, 1, nullptr, cus, stream, -1, false);
}

}  // namespace

extern "C" {

const char* fp8_status_string(fp8_status s) {
    switch (s) {
        case FP8_OK: return "ok";
        case FP8_ERR_INVALID_ARG: return "invalid argument (null pointer, bad dimension or flag)";
        case FP8_ERR_SHAPE: return "unsupported shape (K must be a multiple of 128; grouped N too)";
        case FP8_ERR_ALIGNMENT: return "pointer not 16-byte aligned";
        case FP8_ERR_UNSUPPORTED: return "unsupported configuration";
        case FP8_ERR_NO_DEVICE: return "no usable HIP device";
        case FP8_ERR_LAUNCH: return "kernel launch failed";
        case FP8_ERR_SCRATCH: return "the problem needs more split-K scratch than fp8_gemm_nt_noalloc holds";
    }
    return "unknown status";
}

int32_t fp8_get_mk_alignment_for_contiguous_layout(void) { return 128; }

fp8_status fp8_quant_1x128(const float* x, int64_t M, int64_t K, uint8_t* xq, float* sa,
                           uint32_t flags, void* stream) {
    if (!dims_ok(M) || !dims_ok(K) || (flags & ~FP8_FLAG_UE8M0)) return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (M == 0 || K == 0) return FP8_OK;
    if (!x || !xq || !sa) return FP8_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(xq) || !aligned16(sa)) return FP8_ERR_ALIGNMENT;
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    // one wave per row segment of up to 8 groups, 4 waves per block
    const int64_t units = M * ((K / 128 + 7) / 8);
    const int64_t blocks = (units + 3) / 4;
    if (blocks > 0x7FFFFFFF) return FP8_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (flags & FP8_FLAG_UE8M0)
        hipLaunchKernelGGL(fp8k::quant_1x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0, s,
                           x, xq, sa, M, K, units);
    else
        hipLaunchKernelGGL(fp8k::quant_1x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0, s,
                           x, xq, sa, M, K, units);
    return launch_status();
}

fp8_status fp8_quant_128x128(const float* w, int64_t N, int64_t K, uint8_t* wq, float* sb,
                             uint32_t flags, void* stream) {
    if (!dims_ok(N) || !dims_ok(K) || (flags & ~FP8_FLAG_UE8M0)) return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (N == 0 || K == 0) return FP8_OK;
    if (!w || !wq || !sb) return FP8_ERR_INVALID_ARG;
    if (!aligned16(w) || !aligned16(wq) || !aligned16(sb)) return FP8_ERR_ALIGNMENT;
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    const int64_t blocks = ((N + 127) / 128) * (K / 128);
    if (blocks > 0x7FFFFFFF) return FP8_ERR_INVALID_ARG;
    hipStream_t s = (hipStream_t)stream;
    if (flags & FP8_FLAG_UE8M0)
        hipLaunchKernelGGL(fp8k::quant_128x128_kernel<true>, dim3((unsigned)blocks), dim3(256), 0,
                           s, w, wq, sb, N, K);
    else
        hipLaunchKernelGGL(fp8k::quant_128x128_kernel<false>, dim3((unsigned)blocks), dim3(256), 0,
                           s, w, wq, sb, N, K);
    return launch_status();
}

fp8_status fp8_quant_mx(const float* x, int64_t R, int64_t K, uint8_t* q, uint32_t* e, void* stream) {
    if (!dims_ok(R) || !dims_ok(K)) return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (R == 0 || K == 0) return FP8_OK;
    if (!x || !q || !e) return FP8_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned16(e)) return FP8_ERR_ALIGNMENT;
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    // one wave per row segment of up to 32 groups, 4 waves per block
    const int64_t units = R * ((K / 32 + 31) / 32);
    const int64_t blocks = (units + 3) / 4;
    if (blocks > 0x7FFFFFFF) return FP8_ERR_INVALID_ARG;
    hipLaunchKernelGGL(fp8k::quant_mx_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       x, q, reinterpret_cast<uint8_t*>(e), R, K, units);
    return launch_status();
}

fp8_status fp8_gemm_nt_mx(const uint8_t* xq, const uint32_t* ea, const uint8_t* wq, const uint32_t* eb,
                          uint16_t* y, int64_t M, int64_t N, int64_t K, uint32_t flags, void* stream) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || flags != 0) return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    if (K == 0) return FP8_ERR_SHAPE;
    if (!xq || !ea || !wq || !eb || !y) return FP8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(ea) || !aligned16(eb))
        return FP8_ERR_ALIGNMENT;
    fp8k::GemmParams p{};
    p.xq = xq; p.wq = wq; p.y = y;
    p.sa = reinterpret_cast<const float*>(ea);   // packed scale tables, read as such by the MX path
    p.sb = reinterpret_cast<const float*>(eb);
    p.M = M; p.N = N; p.K = K; p.E = 1;
    return run_gemm_mx<fp8k::kPathMx>(p, (hipStream_t)stream);
}

fp8_status fp8_quant_mxfp4(const float* x, int64_t R, int64_t K, uint8_t* q, uint32_t* e, void* stream) {
    if (!dims_ok(R) || !dims_ok(K)) return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (R == 0 || K == 0) return FP8_OK;
    if (!x || !q || !e) return FP8_ERR_INVALID_ARG;
    if (!aligned16(x) || !aligned16(q) || !aligned16(e)) return FP8_ERR_ALIGNMENT;
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    const int64_t units = R * ((K / 32 + 31) / 32);
    const int64_t blocks = (units + 3) / 4;
    if (blocks > 0x7FFFFFFF) return FP8_ERR_INVALID_ARG;
    hipLaunchKernelGGL(fp8k::quant_mxfp4_kernel, dim3((unsigned)blocks), dim3(256), 0, (hipStream_t)stream,
                       x, q, reinterpret_cast<uint8_t*>(e), R, K, units);
    return launch_status();
}

fp8_status fp8_gemm_nt_mx_w4(const uint8_t* xq, const uint32_t* ea, const uint8_t* wq, const uint32_t* eb,
                             uint16_t* y, int64_t M, int64_t N, int64_t K, uint32_t flags, void* stream) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || flags != 0) return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    if (K == 0) return FP8_ERR_SHAPE;
    if (!xq || !ea || !wq || !eb || !y) return FP8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(ea) || !aligned16(eb))
        return FP8_ERR_ALIGNMENT;
    fp8k::GemmParams p{};
    p.xq = xq; p.wq = wq; p.y = y;
    p.sa = reinterpret_cast<const float*>(ea);
    p.sb = reinterpret_cast<const float*>(eb);
    p.M = M; p.N = N; p.K = K; p.E = 1;
    return run_gemm_mx<fp8k::kPathMxW4>(p, (hipStream_t)stream);
}

fp8_status fp8_gemm_nt_ws(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sb,
                          uint16_t* y, int64_t M, int64_t N, int64_t K, uint32_t flags, void* workspace,
                          size_t workspace_bytes, void* stream) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || (flags & ~kGemmFlags))
        return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    if (K == 0) return FP8_ERR_SHAPE;
    if (!xq || !sa || !wq || !sb || !y || (workspace_bytes && !workspace)) return FP8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(sa) || !aligned16(sb) ||
        !aligned16(workspace))
        return FP8_ERR_ALIGNMENT;
    fp8k::GemmParams p{};
    p.xq = xq; p.sa = sa; p.wq = wq; p.sb = sb; p.y = y;
    p.M = M; p.N = N; p.K = K; p.E = 1;
    return run_gemm<fp8k::kDense>(p, flags, workspace, workspace ? workspace_bytes : 0, (hipStream_t)stream);
}

fp8_status fp8_gemm_nt(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sb,
                       uint16_t* y, int64_t M, int64_t N, int64_t K, uint32_t flags,
                       void* stream) {
    return fp8_gemm_nt_ws(xq, sa, wq, sb, y, M, N, K, flags, nullptr, 0, stream);
}

fp8_status fp8_gemm_nt_noalloc(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sb,
                               uint16_t* y, int64_t M, int64_t N, int64_t K, uint32_t flags, void* stream) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || (flags & ~kGemmFlags))
        return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    const size_t need = fp8_gemm_workspace_size(M, N, K, flags);
    if (need > kScratchBytes) return FP8_ERR_SCRATCH;
    void* ws = nullptr;
    if (need) {
        const fp8_status st = current_device_scratch(&ws);
        if (st != FP8_OK) return st;
    }
    return fp8_gemm_nt_ws(xq, sa, wq, sb, y, M, N, K, flags, ws, need, stream);
}

size_t fp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, uint32_t flags) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || (flags & ~kGemmFlags) || K % 128 || M == 0 || N == 0)
        return 0;
    int cus = 0;
    if (current_device_cus(&cus) != FP8_OK) return 0;
    const Plan pl = make_plan(fp8k::kDense, M, N, K, flags, false, false, cus, SIZE_MAX);
    return (pl.main == kFastDecode || pl.main == kExactDecode || pl.main == kExactDecodeX) && pl.k_splits > 1
               ? decode_ws_bytes(pl.k_splits, M, N) : 0;
}

fp8_status fp8_gemm_plan(int32_t layout, int64_t M, int64_t N, int64_t K, uint32_t flags, int32_t compute_units,
                         size_t workspace_bytes, fp8_gemm_plan_t* plan) {
    const uint32_t known = kGemmFlags | FP8_PLAN_MX | FP8_PLAN_QOUT;
    if (!plan || layout < 0 || layout > 2 || !dims_ok(M) || !dims_ok(N) || !dims_ok(K) || compute_units <= 0 ||
        (flags & ~known))
        return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    const bool mx = flags & FP8_PLAN_MX, qout = flags & FP8_PLAN_QOUT;
    if ((mx || qout) && layout != 0) return FP8_ERR_INVALID_ARG;
    const Plan pl = make_plan(layout, M, N, K, flags & kGemmFlags, mx, qout, compute_units, workspace_bytes);
    const InstInfo a = inst_info(pl.main);
    *plan = fp8_gemm_plan_t{};
    plan->exact = a.exact;
    plan->kernel = a.kernel;
    plan->tile_m = a.bm;
    plan->tile_n = a.bn;
    plan->waves = a.waves;
    plan->main_rows = layout == 1 ? pl.main_rows : M;
    plan->main_cols = layout == 0 && pl.main_cols > 0 ? pl.main_cols : N;
    plan->k_splits = (int32_t)pl.k_splits;
    plan->workspace_bytes = pl.k_splits > 1 ? decode_ws_bytes(pl.k_splits, M, N) : 0;
    if (a.kernel != 0) {
        plan->tiles = cdiv(N, a.bn) * pl.k_splits;
        plan->grid = (int32_t)plan->tiles;
    } else {
        const int64_t rows = layout == 1 ? pl.main_rows : M;
        const int64_t cols = layout == 0 && pl.main_cols > 0 ? pl.main_cols : N;
        plan->tiles = cdiv(rows, a.bm) * cdiv(cols, a.bn);
        // the masked launches have one workgroup per possible tile
        const bool per_tile = layout == 2;
        plan->grid = (int32_t)(plan->tiles < compute_units || per_tile ? plan->tiles : compute_units);
    }
    if (layout == 1 && pl.paired) {
        // the shares of the three launches are found on the device: upper bounds
        const InstInfo m = inst_info(pl.mid), t = inst_info(pl.tail);
        plan->paired = 1;
        plan->mid_tile_m = m.bm;
        plan->mid_tile_n = m.bn;
        plan->mid_tiles = cdiv(M, m.bm) * cdiv(N, m.bn);
        plan->tail_tile_m = t.bm;
        plan->tail_tile_n = t.bn;
        plan->tail_tiles = cdiv(M, t.bm) * cdiv(N, t.bn);
    } else if (layout == 1 && pl.main_rows < M) {
        const InstInfo t = inst_info(pl.tail);
        plan->tail_tile_m = t.bm;
        plan->tail_tile_n = t.bn;
        plan->tail_tiles = cdiv(M - pl.main_rows, t.bm) * cdiv(N, t.bn);
    }
    if (layout == 0 && pl.main_cols > 0 && pl.main_cols < N) {
        const InstInfo t = inst_info(pl.tail);
        plan->tail_tile_m = t.bm;
        plan->tail_tile_n = t.bn;
        plan->tail_tiles = cdiv(M, t.bm) * cdiv(N - pl.main_cols, t.bn);
    }
    return FP8_OK;
}

fp8_status fp8_gemm_nt_qout(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sb,
                            uint8_t* yq, float* sy, int64_t M, int64_t N, int64_t K, uint32_t flags,
                            void* stream) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || (flags & ~kGemmFlags))
        return FP8_ERR_INVALID_ARG;
    if (K % 128 || N % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    if (K == 0) return FP8_ERR_SHAPE;
    if (!xq || !sa || !wq || !sb || !yq || !sy) return FP8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(sa) || !aligned16(sb) || !aligned16(yq) ||
        !aligned16(sy))
        return FP8_ERR_ALIGNMENT;
    fp8k::GemmParams p{};
    p.xq = xq; p.sa = sa; p.wq = wq; p.sb = sb; p.yq = yq; p.sy = sy;
    p.M = M; p.N = N; p.K = K; p.E = 1;
    return run_gemm<fp8k::kDense>(p, flags, nullptr, 0, (hipStream_t)stream, true);
}

fp8_status fp8_grouped_gemm_contiguous(const uint8_t* xq, const float* sa, const uint8_t* wq,
                                       const float* sb, const int32_t* m_indices, uint16_t* y,
                                       int64_t M, int64_t N, int64_t K, int32_t E,
                                       uint32_t flags, void* stream) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || E < 0 || (flags & ~kGemmFlags))
        return FP8_ERR_INVALID_ARG;
    if (K % 128 || N % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0 || E == 0) return FP8_OK;
    if (K == 0) return FP8_ERR_SHAPE;
    if (!xq || !sa || !wq || !sb || !m_indices || !y) return FP8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(sa) || !aligned16(sb) ||
        !aligned16(m_indices))
        return FP8_ERR_ALIGNMENT;
    fp8k::GemmParams p{};
    p.xq = xq; p.sa = sa; p.wq = wq; p.sb = sb; p.y = y; p.m_indices = m_indices;
    p.M = M; p.N = N; p.K = K; p.E = E;
    return run_gemm<fp8k::kContiguous>(p, flags, nullptr, 0, (hipStream_t)stream);
}

fp8_status fp8_grouped_gemm_masked(const uint8_t* xq, const float* sa, const uint8_t* wq,
                                   const float* sb, const int32_t* masked_m, uint16_t* y,
                                   int32_t E, int64_t max_m, int64_t N, int64_t K,
                                   uint32_t flags, void* stream) {
    if (E < 0 || !dims_ok(max_m) || !dims_ok(N) || !dims_ok(K) ||
        !dims_ok((int64_t)E * max_m) || (flags & ~kGemmFlags))
        return FP8_ERR_INVALID_ARG;
    if (K % 128 || N % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (E == 0 || max_m == 0 || N == 0) return FP8_OK;
    if (K == 0) return FP8_ERR_SHAPE;
    if (!xq || !sa || !wq || !sb || !masked_m || !y) return FP8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(sa) || !aligned16(sb) ||
        !aligned16(masked_m))
        return FP8_ERR_ALIGNMENT;
    fp8k::GemmParams p{};
    p.xq = xq; p.sa = sa; p.wq = wq; p.sb = sb; p.y = y; p.masked_m = masked_m;
    p.M = (int64_t)E * max_m; p.N = N; p.K = K; p.E = E; p.max_m = max_m;
    return run_gemm<fp8k::kMasked>(p, flags, nullptr, 0, (hipStream_t)stream);
}

}  // extern "C"
