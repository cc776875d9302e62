// fp8gemm_api.hip -- host side of libfp8gemm.so: argument validation, kernel
// instance choice and launches for the C ABI declared in include/fp8gemm.h.
//
// Every entry point validates on the host first and enqueues nothing on an
// error; then it launches asynchronously on the caller's stream.  Nothing is
// allocated, freed or synchronized here.
#include <hip/hip_runtime.h>

#include <atomic>
#include <map>
#include <mutex>
#include <utility>

#include "../../include/fp8gemm.h"
#include "kernels_decode.h"
#include "kernels_gemm.h"
#include "kernels_quant.h"

namespace {

constexpr int64_t kMaxDim = (int64_t)1 << 31;     // rows/cols fit int32 tile math
constexpr int kMaxDevices = 64;
constexpr uint32_t kGemmFlags = FP8_FLAG_UE8M0 | FP8_FLAG_PRECISE;
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

fp8_status launch_status() {
    return hipGetLastError() == hipSuccess ? FP8_OK : FP8_ERR_LAUNCH;
}

// ---------------------------------------------------------------------------
// GEMM instances.  Naming: BM x BN workgroup tile, WAVES_M x WAVES_N waves.
// ---------------------------------------------------------------------------
template <int BM, int BN, int WM, int WN, int MODE, int PATH, int STAGES = 2, int GROUP_M = 4,
          bool QOUT = false>
fp8_status launch_gemm(fp8k::GemmParams p, int cus, hipStream_t stream, int64_t m_hi = -1) {
    // dense/contiguous: tiles over rows [p.m_lo, m_hi) (all rows by default)
    if (m_hi < 0) m_hi = p.M;
    p.m_tiles = (int)((MODE == fp8k::kMasked ? p.max_m : m_hi - p.m_lo) + BM - 1) / BM;
    p.n_tiles = (int)((p.N + BN - 1) / BN);
    p.group_m = GROUP_M;
    int64_t tiles = (int64_t)p.m_tiles * p.n_tiles;
    if (MODE == fp8k::kMasked) tiles *= p.E;   // upper bound; the kernel counts the real ones
    int grid = (int)(tiles < cus ? tiles : cus);
    if (grid <= 0) return FP8_OK;
    hipLaunchKernelGGL((fp8k::gemm_kernel<BM, BN, WM, WN, MODE, PATH, STAGES, QOUT>), dim3(grid),
                       dim3(64 * WM * WN), 0, stream, p.xq, p.sa, p.wq, p.sb, p.y, p.m_indices,
                       p.masked_m, p);
    return launch_status();
}

// Decode-sized dense GEMM (M <= 32): one workgroup per 16*NW output columns
// and all M rows, one wave per 16 columns; MSUB = ceil(M/16) row subtiles.
// With fewer column tiles than compute units the K chunks are split over up
// to 8 workgroups per tile (one workgroup per CU in all): they write FP32
// partial sums to the stream's split workspace and a second kernel adds them
// in split order and rounds to BF16.  Without a workspace the GEMM runs
// unsplit.
// Split-K workspace of the decode GEMM: one buffer per (device, stream),
// sized for the largest split the device takes (8 splits x 32 rows x fewer
// than 96*CUs columns of FP32), allocated on first use and kept until the
// process ends.  Calls on one stream are ordered, so they can share it; other
// streams have their own.  Nothing is allocated while the stream is being
// captured into a graph, nor past kMaxSplitWorkspaces buffers in the process
// (a caller that makes a new stream per call would otherwise add one per
// stream): the GEMM then runs unsplit.
constexpr size_t kMaxSplitWorkspaces = 16;
std::mutex g_split_mu;
std::map<std::pair<int, hipStream_t>, void*> g_split_ws;

size_t split_ws_bytes(int cus) { return (size_t)8 * 32 * 96 * (size_t)cus * sizeof(float); }

void* split_workspace(int cus, hipStream_t stream) {
    int dev = -1;
    if (hipGetDevice(&dev) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    std::lock_guard<std::mutex> lock(g_split_mu);
    const auto key = std::make_pair(dev, stream);
    const auto it = g_split_ws.find(key);
    if (it != g_split_ws.end()) return it->second;
    if (g_split_ws.size() >= kMaxSplitWorkspaces) return nullptr;
    hipStreamCaptureStatus cap = hipStreamCaptureStatusNone;
    if (hipStreamIsCapturing(stream, &cap) != hipSuccess || cap != hipStreamCaptureStatusNone) {
        (void)hipGetLastError();
        return nullptr;
    }
    void* ws = nullptr;
    if (hipMalloc(&ws, split_ws_bytes(cus)) != hipSuccess) {
        (void)hipGetLastError();
        return nullptr;
    }
    g_split_ws[key] = ws;
    return ws;
}

template <int NW, int NS, bool POW2>
fp8_status launch_decode(const fp8k::GemmParams& p0, int cus, hipStream_t stream) {
    fp8k::GemmParams p = p0;
    const int64_t tiles = (p.N + 16 * NW - 1) / (16 * NW);
    if (tiles <= 0) return FP8_OK;
    const int64_t nct = (p.K / 128 + 3) / 4;          // K chunks of 4 blocks
    int64_t splits = tiles < cus ? cus / tiles : 1;
    if (splits > nct) splits = nct;
    if (splits > 8) splits = 8;
    if (splits < 1) splits = 1;
    void* ws = nullptr;
    if (splits > 1) {
        // splits <= 8, M <= 32, N < 96 * cus: the buffer always holds them
        ws = (size_t)(splits * p.M * p.N) * sizeof(float) <= split_ws_bytes(cus) ? split_workspace(cus, stream)
                                                                                : nullptr;
        if (!ws) splits = 1;
    }
    p.part = static_cast<float*>(ws);
    const dim3 grid((unsigned)tiles, (unsigned)splits), block(64 * NW);
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
        hipLaunchKernelGGL(fp8k::decode_split_reduce, dim3((unsigned)((mn + 255) / 256)), dim3(256), 0, stream,
                           static_cast<const float*>(ws), (int)splits, mn, p.y);
        st = launch_status();
    }
    return st;
}

// Decode-sized dense GEMM with 32 < M <= 48 and K <= kDecodeKxMaxK: X resident
// in LDS, waves splitting K.
template <bool POW2>
fp8_status launch_decode_kx(const fp8k::GemmParams& p, hipStream_t stream) {
    const int64_t tiles = (p.N + 95) / 96;
    if (tiles <= 0) return FP8_OK;
    hipLaunchKernelGGL((fp8k::decode_kx_kernel<3, POW2>), dim3((unsigned)tiles), dim3(512), 0, stream,
                       p.xq, p.sa, p.wq, p.sb, p.y, p);
    return launch_status();
}

// Instances.  Compute-bound shapes use 8 waves (2 per SIMD) so that one wave's
// promotion FMAs run while the other wave's MFMAs occupy the matrix core.
template <int MODE, int PATH>
fp8_status dispatch_gemm(const fp8k::GemmParams& p, int cus, hipStream_t stream) {
    if constexpr (MODE == fp8k::kDense) {
        if (p.M <= 64) {
            // FP8 MFMA paths.  M <= 32: the decode kernel (96 columns per
            // workgroup, one wave per 16 W rows).  Above 32 rows each of its
            // waves re-reads an X block larger than its W block from LDS;
            // 33..48 rows with K <= 1664 take the X-resident decode kernel
            // (waves splitting K), and the rest the 64x96 tile of the main
            // kernel.  Kernel trace, N 24576, K 1536: M 16 7.3 vs 10.3 us
            // (64x96), M 32 8.8 vs 10.3, M 48 9.6 (X-resident) vs 10.4, M 64
            // 10.7 (X-resident) and 12.2 (decode) vs 10.0-10.4.  A 32-column
            // decode workgroup (more of them, several per CU) measured slower
            // on every shape tried.
            if constexpr (PATH == fp8k::kPathFp8 || PATH == fp8k::kPathFp8Pow2) {
                if (p.M <= 32) return launch_decode<6, 5, PATH == fp8k::kPathFp8Pow2>(p, cus, stream);
                if (p.M <= 48 && p.K <= fp8k::kDecodeKxMaxK)
                    return launch_decode_kx<PATH == fp8k::kPathFp8Pow2>(p, stream);
            }
            return launch_gemm<64, 96, 2, 2, MODE, PATH, 3>(p, cus, stream);
        }
        constexpr bool kF16 = PATH == fp8k::kPathF16 || PATH == fp8k::kPathF16Pow2;
        const int64_t huge = ((p.M + 255) / 256) * ((p.N + 255) / 256);
        if constexpr (!kF16) {
            if (huge >= cus) {
                // 256x224 when it takes fewer waves' worth of tile area (e.g.
                // N = 7168: 32 tiles of 224 per row fill two whole waves where
                // 28 tiles of 256 leave the second one a quarter empty)
                const int64_t t224 = ((p.M + 255) / 256) * ((p.N + 223) / 224);
                const int64_t cost256 = ((huge + cus - 1) / cus) * 256;
                const int64_t cost224 = ((t224 + cus - 1) / cus) * 224;
                if (cost224 < cost256) return launch_gemm<256, 224, 4, 2, MODE, PATH>(p, cus, stream);
                return launch_gemm<256, 256, 2, 4, MODE, PATH>(p, cus, stream);
            }
        }
        const int64_t big = ((p.M + 255) / 256) * ((p.N + 127) / 128);
        if (big >= 2 * cus || (kF16 && huge >= cus)) return launch_gemm<256, 128, 4, 2, MODE, PATH, 3>(p, cus, stream);
        return launch_gemm<128, 128, 2, 2, MODE, PATH, 4>(p, cus, stream);
    } else if constexpr (MODE == fp8k::kContiguous) {
        // The M tile must equal the layout alignment (128): one expert per tile.
        // When the last round of 128x256 tiles would leave over half of the
        // CUs idle, the full rounds' 128-row blocks run as one launch and the
        // remaining blocks as a second one with 128x64 tiles (8 waves of
        // 32x32), four times as many (8 experts x 8192 tokens, N 4096: 1088
        // tiles = 4.25 rounds -> 4 full rounds + 256 tiles of 128x64; measured
        // 343 -> 327 us).
        const int64_t mt = (p.M + 127) / 128, nt = (p.N + 255) / 256;
        const int64_t full = mt * nt / cus, last = mt * nt - full * cus;
        const int64_t m_main = full * cus / nt;   // 128-row blocks of the full rounds
        if (full >= 1 && 2 * last < cus && m_main < mt) {
            fp8_status st = launch_gemm<128, 256, 2, 4, MODE, PATH, 3>(p, cus, stream, m_main * 128);
            if (st != FP8_OK) return st;
            fp8k::GemmParams t = p;
            t.m_lo = m_main * 128;
            return launch_gemm<128, 64, 4, 2, MODE, PATH, 4>(t, cus, stream);
        }
        return launch_gemm<128, 256, 2, 4, MODE, PATH, 3>(p, cus, stream);
    } else {
        // Masked: 128-row tiles pad each expert's rows less than 256-row ones,
        // and 256 columns per tile halve the re-reads of the expert's X rows
        // (measured 94 -> 82 us on 16 experts x 256 rows, N 7168, K 2048).
        return launch_gemm<128, 256, 2, 4, MODE, PATH, 3>(p, cus, stream);
    }
}

// Quantized-output instances: 128-column output groups need a tile width of
// 128 or 256 with 64-column waves (no 256x224, no 64x96).
template <int PATH>
fp8_status dispatch_qout(const fp8k::GemmParams& p, int cus, hipStream_t stream) {
    constexpr bool kF16 = PATH == fp8k::kPathF16 || PATH == fp8k::kPathF16Pow2;
    const int64_t huge = ((p.M + 255) / 256) * ((p.N + 255) / 256);
    if constexpr (!kF16)
        if (huge >= cus) return launch_gemm<256, 256, 2, 4, fp8k::kDense, PATH, 2, 4, true>(p, cus, stream);
    const int64_t big = ((p.M + 255) / 256) * ((p.N + 127) / 128);
    if (big >= 2 * cus || (kF16 && huge >= cus))
        return launch_gemm<256, 128, 4, 2, fp8k::kDense, PATH, 3, 4, true>(p, cus, stream);
    return launch_gemm<128, 128, 2, 2, fp8k::kDense, PATH, 4, 4, true>(p, cus, stream);
}

fp8_status run_gemm_qout(const fp8k::GemmParams& p, uint32_t flags, hipStream_t stream) {
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    const bool pow2 = flags & FP8_FLAG_UE8M0, precise = flags & FP8_FLAG_PRECISE;
    if (precise)
        return pow2 ? dispatch_qout<fp8k::kPathF16Pow2>(p, cus, stream)
                    : dispatch_qout<fp8k::kPathF16>(p, cus, stream);
    return pow2 ? dispatch_qout<fp8k::kPathFp8Pow2>(p, cus, stream)
                : dispatch_qout<fp8k::kPathFp8>(p, cus, stream);
}

template <int MODE>
fp8_status run_gemm(const fp8k::GemmParams& p, uint32_t flags, hipStream_t stream) {
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    const bool pow2 = flags & FP8_FLAG_UE8M0, precise = flags & FP8_FLAG_PRECISE;
    if (precise)
        return pow2 ? dispatch_gemm<MODE, fp8k::kPathF16Pow2>(p, cus, stream)
                    : dispatch_gemm<MODE, fp8k::kPathF16>(p, cus, stream);
    return pow2 ? dispatch_gemm<MODE, fp8k::kPathFp8Pow2>(p, cus, stream)
                : dispatch_gemm<MODE, fp8k::kPathFp8>(p, cus, stream);
}

bool dims_ok(int64_t a) { return a >= 0 && a < kMaxDim; }

// MXFP8: the dense instance table with the MX path (scales as per-lane E8M0
// operands, no promotion).
fp8_status run_gemm_mx(const fp8k::GemmParams& p, hipStream_t stream) {
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    return dispatch_gemm<fp8k::kDense, fp8k::kPathMx>(p, cus, stream);
}

fp8_status run_gemm_mx_w4(const fp8k::GemmParams& p, hipStream_t stream) {
    int cus = 0;
    fp8_status st = current_device_cus(&cus);
    if (st != FP8_OK) return st;
    return dispatch_gemm<fp8k::kDense, fp8k::kPathMxW4>(p, cus, stream);
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
    return run_gemm_mx(p, (hipStream_t)stream);
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
    return run_gemm_mx_w4(p, (hipStream_t)stream);
}

fp8_status fp8_gemm_nt(const uint8_t* xq, const float* sa, const uint8_t* wq, const float* sb,
                       uint16_t* y, int64_t M, int64_t N, int64_t K, uint32_t flags,
                       void* stream) {
    if (!dims_ok(M) || !dims_ok(N) || !dims_ok(K) || (flags & ~kGemmFlags))
        return FP8_ERR_INVALID_ARG;
    if (K % 128) return FP8_ERR_SHAPE;
    if (K > kMaxGemmK) return FP8_ERR_UNSUPPORTED;
    if (M == 0 || N == 0) return FP8_OK;
    if (K == 0) return FP8_ERR_SHAPE;
    if (!xq || !sa || !wq || !sb || !y) return FP8_ERR_INVALID_ARG;
    if (!aligned16(xq) || !aligned16(wq) || !aligned16(y) || !aligned16(sa) || !aligned16(sb))
        return FP8_ERR_ALIGNMENT;
    fp8k::GemmParams p{};
    p.xq = xq; p.sa = sa; p.wq = wq; p.sb = sb; p.y = y;
    p.M = M; p.N = N; p.K = K; p.E = 1;
    return run_gemm<fp8k::kDense>(p, flags, (hipStream_t)stream);
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
    return run_gemm_qout(p, flags, (hipStream_t)stream);
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
    return run_gemm<fp8k::kContiguous>(p, flags, (hipStream_t)stream);
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
    return run_gemm<fp8k::kMasked>(p, flags, (hipStream_t)stream);
}

}  // extern "C"
