// kernels_decode.h -- block-scaled E4M3 NT GEMM for decode-sized M on gfx950:
// decode_kernel (M <= 32, optionally split over K) with its split-K reduction,
// and decode_kx_kernel (32 < M <= 48, X resident in LDS).
//
// Same result as gemm_kernel: Y[m][n] = sum_kb sa[kb][m] * sb[n/128][kb] *
// P_kb[m][n], each 128-K block partial P_kb formed by one FP8 MFMA and
// promoted into an FP32 accumulator (tcgen05 page, section 6.1; DeepGEMM
// page, "主循环骨架").  With so few rows the GEMM is a stream of W: every W
// byte is used by at most 64 rows, far below the matrix core's ratio of FLOPs
// to HBM bytes, so the time is the HBM read of W (tcgen05 page, sections 5.4
// and 8.2: small-batch decode is bandwidth-bound and wants a shape-specific
// kernel rather than the large-tile main loop).
//
// gfx950 mapping
//   * A workgroup owns TN = 16*NW consecutive W rows (output columns) and all
//     M rows of X; each of its NW waves owns one 16-row subtile of W over the
//     whole of K, so no partial sums cross waves.
//   * W streams through a private LDS ring per wave: a 16-row x 128-byte K
//     block is two direct-to-LDS loads of eight full 128-byte rows each (a
//     wave instruction covering whole rows reads HBM at the full rate, where
//     the MFMA operand layout -- 64 bytes of each of 16 rows -- does not), the
//     loads run NS-1 blocks ahead, and the wave waits only on its own
//     vector-memory counter: no barrier per K block.
//   * X and the scales are shared by the waves: they arrive in chunks of
//     KBC = 4 K blocks, double-buffered in LDS, loaded by all waves together
//     one chunk ahead; one barrier per chunk publishes a chunk and frees the
//     buffer of the one before.  Row stride of an X chunk in LDS: 640 bytes
//     (an odd multiple of 128), with the 16-byte chunk c of row r at slot
//     c ^ lds_swz(r) as in every LDS tile here, so that fragment reads of 16
//     rows hit distinct bank groups.
//   * Every load is an LDS DMA issued in a fixed order, so each wait is a
//     compile-time count of the loads issued after the one waited for (loads
//     past the end of K go through an empty buffer range: issued and counted,
//     but they touch no memory).
//   * Fragment K order: lane group g (lanes 16g .. 16g+15) holds bytes
//     16g .. 16g+15 and 64+16g .. 64+16g+15 of its row's K block, the same
//     order for both operands (a dot product does not depend on how K is
//     ordered as long as both operands agree).
//   * W is the MFMA A operand and X the B operand: lane l of a 16x16 result
//     holds n = 4*(l/16) + r (r = 0..3) of column m = l%16, so each lane has
//     one sA per m subtile and the wave's 16 n share one sB (a 16-row subtile
//     never straddles a 128-row weight block).
//   * Power-of-two scales (UE8M0): they are the E8M0 operands of the scaled
//     MFMA and K accumulates inside the matrix core.
//   * Split K (grid.y > 1, chosen by the host when the column tiles are fewer
//     than the CUs): workgroup (t, s) takes a contiguous range of the K chunks
//     and writes FP32 partial sums [s][M][N]; decode_split_reduce adds them in
//     split order and rounds to BF16.
#pragma once

#include "device_common.h"
#include "kernels_gemm.h"

namespace fp8k {

template <int MSUB, int NW, int NS>
struct DecodeLayout {
    static constexpr int KBC = 4;                      // K blocks per X chunk
    static constexpr int XSTRIDE = 640;                // LDS bytes per X row of a chunk
    static constexpr int MR = 16 * MSUB;               // X rows staged (rows past M read zeros)
    static constexpr int XBYTES = MR * XSTRIDE;        // one X chunk
    static constexpr int NXL = XBYTES / 1024;          // its 1 KB loads
    static constexpr int NSA = KBC * MR * 4 / 256;     // dword loads of the chunk's sA
    static constexpr int NT = NXL + NSA + 1;           // + one dword load of its sB
    static constexpr int NPW = (NT + NW - 1) / NW;     // chunk loads per wave (the same for every wave)
    static constexpr int X0 = 0;                       // X chunk buffers
    static constexpr int SA0 = 2 * XBYTES;             // sA [KBC][MR] floats, two buffers
    static constexpr int SB0 = SA0 + 2 * KBC * MR * 4; // sB [2][KBC] floats (64 lanes' worth), two buffers
    static constexpr int W0 = SB0 + 2 * 256;           // W rings: [wave][stage] 2 KB
    static constexpr int SPARE = W0 + NW * NS * 2048;  // target of the surplus chunk loads
    static constexpr int BYTES = SPARE + 1024;
    static_assert(XBYTES % 1024 == 0 && (KBC * MR * 4) % 256 == 0, "whole wave loads");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

template <int MSUB, int NW, int NS, bool POW2>
__global__ __launch_bounds__(64 * NW, 1) void decode_kernel(
    const uint8_t* __restrict__ xq_, const float* __restrict__ sa_, const uint8_t* __restrict__ wq_,
    const float* __restrict__ sb_, uint16_t* __restrict__ y_, GemmParams p) {
    using L = DecodeLayout<MSUB, NW, NS>;
    constexpr int KBC = L::KBC, D = NS - 1, NPW = L::NPW;
    // the wait counts below assume the W loads of a block are issued at most
    // one chunk ahead of its use
    static_assert(MSUB >= 1 && MSUB <= 4 && NW >= 1 && NS >= 2 && D <= KBC, "decode tile");
    static_assert(2 * D + NPW <= 63 && 2 * KBC <= 63, "vmcnt range");
    constexpr int TN = 16 * NW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::BYTES];

    const int lane = threadIdx.x & 63;
    const int w = uniform(threadIdx.x >> 6);
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int KB = (int)(K >> 7);
    // Split K (grid.y > 1, for few column tiles): this workgroup takes the
    // chunks [cs0, cs0 + NC) of the K range and writes FP32 partial sums.
    const int NCT = (KB + KBC - 1) / KBC;
    const int cs0 = (int)(blockIdx.y * NCT / gridDim.y);
    const int NC = (int)((blockIdx.y + 1) * NCT / gridDim.y) - cs0;
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    const int64_t nw = n0 + 16 * w;                   // this wave's first column
    const uint32_t lds0 = lds_addr(smem);

    // Buffer resources: rows past the matrix edges read zeros.
    const int64_t rows_w = N - n0 < TN ? N - n0 : TN;
    const i32x4 wr = make_rsrc(wq_ + n0 * K, (uint32_t)(rows_w * K));
    const i32x4 xr = make_rsrc(xq_, (uint32_t)(M * K));
    const i32x4 sar = make_rsrc(sa_, (uint32_t)(KB * M * 4));
    const int64_t nb0 = n0 >> 7, nb1 = (n0 + rows_w - 1) >> 7;
    const i32x4 sbr = make_rsrc(sb_ + nb0 * KB, (uint32_t)((nb1 - nb0 + 1) * KB * 4));
    const i32x4 none = make_rsrc(wq_, 0u);
    constexpr uint32_t kFar = 0x7FFFFFF0u;              // an offset past every range

    // ---- W: this wave's 16 rows, two 1 KB loads per K block ----
    // load h, lane l: row 8h + l/8, LDS slot l%8 holding logical chunk
    // (l%8) ^ lds_swz(row)
    uint32_t wsrc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + (lane >> 3);
        wsrc[h] = (uint32_t)((16 * w + r) * K) + 16 * ((lane & 7) ^ lds_swz(r));
    }
    const uint32_t wring = lds0 + L::W0 + (uint32_t)w * NS * 2048;
    // K block of sequence position q (past the end: KB, loaded empty)
    auto seq_kb = [&](int q) -> int {
        const int c = q / KBC;
        if (c >= NC) return KB;
        return (cs0 + c) * KBC + (q - c * KBC);
    };
    auto issue_w = [&](int q) {
        const int kb = seq_kb(q);
        const bool in = kb < KB;
        const i32x4 rs = in ? wr : none;
        const uint32_t dst = wring + (uint32_t)(q % NS) * 2048;
        dma_lds16_one<0>(dst, wsrc[0] + (in ? kb : 0) * 128, rs, 0);
        dma_lds16_one<0>(dst + 1024, wsrc[1] + (in ? kb : 0) * 128, rs, 0);
    };

    // ---- X, sA, sB of chunk c: NPW loads per wave, slot i = w + NW*t ----
    auto issue_chunk = [&](int c) {
        const bool in = c < NC;
        const int buf = c & 1;
        const int cd = cs0 + c;                        // data chunk
        const int k0 = cd * KBC * 128, kb0 = cd * KBC;
#pragma unroll
        for (int t = 0; t < NPW; ++t) {
            const int i = w + NW * t;                  // wave-uniform
            if (i < L::NXL) {
                const int d = 1024 * i + 16 * lane;
                const int r = d / L::XSTRIDE, j = (d - r * L::XSTRIDE) >> 4;
                const int cc = j ^ lds_swz(r);
                const uint32_t src = (in && j < 8 * KBC) ? (uint32_t)(r * K + k0 + 16 * cc) : kFar;
                dma_lds16_one<0>(lds0 + L::X0 + buf * L::XBYTES + 1024 * i, src, in ? xr : none, 0);
            } else if (i < L::NXL + L::NSA) {
                const int f = 64 * (i - L::NXL) + lane;     // float f of the chunk's [KBC][MR] sA
                const int kb = f / L::MR, m = f - kb * L::MR;
                const uint32_t src = (in && m < M) ? (uint32_t)(((kb0 + kb) * M + m) * 4) : kFar;
                dma_lds4(lds0 + L::SA0 + buf * (KBC * L::MR * 4) + 256 * (i - L::NXL), src, in ? sar : none, 0);
            } else if (i < L::NT) {
                // lane b*KBC + kb: sB of weight block nb0 + b, K block kb0 + kb
                const int b = lane / KBC, kb = lane - b * KBC;
                const uint32_t src = (in && b < 2) ? (uint32_t)((b * KB + kb0 + kb) * 4) : kFar;
                dma_lds4(lds0 + L::SB0 + buf * 256, src, in ? sbr : none, 0);
            } else {
                dma_lds16_one<0>(lds0 + L::SPARE, kFar, none, 0);
            }
        }
    };

    // ---- fragment reads ----
    const int sw = lds_swz(r16);
    const uint32_t wfa = (uint32_t)r16 * 128 + 16 * (g ^ sw), wfb = (uint32_t)r16 * 128 + 16 * ((4 + g) ^ sw);
    const uint32_t xfa = (uint32_t)r16 * L::XSTRIDE + 16 * (g ^ sw);
    const uint32_t xfb = (uint32_t)r16 * L::XSTRIDE + 16 * ((4 + g) ^ sw);
    const int sbl = (int)((nw >> 7) - nb0);            // this wave's weight block in the chunk's sB
    auto rd16 = [&](uint32_t off) -> i32x4 { return *reinterpret_cast<const i32x4*>(smem + off); };

    f32x4 acc[MSUB];
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms) acc[ms] = f32x4{0.f, 0.f, 0.f, 0.f};

    auto compute = [&](int q, int buf, int kbl) {
        const uint32_t ws = L::W0 + (uint32_t)w * NS * 2048 + (uint32_t)(q % NS) * 2048;
        const i32x4 wa = rd16(ws + wfa), wb = rd16(ws + wfb);
        const i32x8 wf = i32x8{wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
        const float sbv = *reinterpret_cast<const float*>(smem + L::SB0 + buf * 256 + 4 * (sbl * KBC + kbl));
        const uint32_t xs = L::X0 + buf * L::XBYTES + 128 * kbl;
        const float* sap = reinterpret_cast<const float*>(smem + L::SA0 + buf * (KBC * L::MR * 4)) + kbl * L::MR + r16;
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) {
            const i32x4 xa = rd16(xs + ms * 16 * L::XSTRIDE + xfa), xb = rd16(xs + ms * 16 * L::XSTRIDE + xfb);
            const i32x8 xf = i32x8{xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            const float sav = sap[16 * ms];
            if constexpr (POW2) {
                acc[ms] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(wf, xf, acc[ms], 0, 0, 0, e8m0_of(sbv),
                                                                           0, e8m0_of(sav));
            } else {
                const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                    wf, xf, f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                const float sc = sav * sbv;
#pragma unroll
                for (int r = 0; r < 4; ++r) acc[ms][r] = __builtin_fmaf(sc, part[r], acc[ms][r]);
            }
        }
    };

    // ---- issue order and waits ----
    // prologue: chunk 0, then the W blocks of positions 0 .. D-1
    issue_chunk(0);
#pragma unroll
    for (int j = 0; j < D; ++j) issue_w(j);
    for (int c = 0; c < NC; ++c) {
        // this wave's part of chunk c: issued before the D prologue W blocks
        // (c = 0) or before the KBC W blocks of the previous chunk's positions
        if (c == 0) wait_vmcnt<2 * D>();
        else wait_vmcnt<2 * KBC>();
        // chunk c published; this wave's reads of chunk c-1 complete before
        // the barrier, after which its buffer is refilled
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue_chunk(c + 1);
        static_for<KBC>([&](auto pc) {
            constexpr int pos = decltype(pc)::value;
            const int q = c * KBC + pos;               // sequence position
            // position q+D reuses the ring slot of position q-1: this wave's
            // reads of it must have completed (the compiler may sink their
            // MFMAs, and with them the wait for the reads, below this point)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue_w(q + D);
            // loads issued after position q's W block: the next D W blocks,
            // and chunk c+1 when position q's block was issued before it
            wait_vmcnt<2 * D + (pos < D ? NPW : 0)>();
            asm volatile("" ::: "memory");
            if (seq_kb(q) < KB) compute(q, c & 1, pos);
        });
    }
    wait_vmcnt<0>();

    // ---- stores: lane holds n = nw + 4g + r, m = 16 ms + r16 ----
    const int64_t n = nw + 4 * g;
    if (n < N && p.part) {
        // FP32 partial sums of this K range, [split][M][N]
        float* base = p.part + (int64_t)blockIdx.y * M * N;
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) {
            const int64_t m = 16 * ms + r16;
            if (m >= M) continue;
            float* prow = base + m * N;
            if ((N & 3) == 0 && n + 3 < N) {
                *reinterpret_cast<f32x4*>(prow + n) = acc[ms];
            } else {
#pragma unroll
                for (int r = 0; r < 4; ++r)
                    if (n + r < N) prow[n + r] = acc[ms][r];
            }
        }
    } else if (n < N) {
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) {
            const int64_t m = 16 * ms + r16;
            if (m >= M) continue;
            uint16_t* yrow = y_ + m * N;
            const uint32_t lo = pack_bf16x2(acc[ms][0], acc[ms][1]);
            const uint32_t hi = pack_bf16x2(acc[ms][2], acc[ms][3]);
            if ((N & 3) == 0 && n + 3 < N) {
                *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
            } else {
                yrow[n] = (uint16_t)(lo & 0xFFFF);
                if (n + 1 < N) yrow[n + 1] = (uint16_t)(lo >> 16);
                if (n + 2 < N) yrow[n + 2] = (uint16_t)(hi & 0xFFFF);
                if (n + 3 < N) yrow[n + 3] = (uint16_t)(hi >> 16);
            }
        }
    }
}

}  // namespace fp8k

namespace fp8k {

// Split-K reduction of the decode GEMM: Y = BF16(sum over the splits, in
// split order, of the FP32 partial sums [S][M][N]).
__global__ __launch_bounds__(256) void decode_split_reduce(const float* __restrict__ part, int S, int64_t MN,
                                                           uint16_t* __restrict__ y) {
    const int64_t i = (int64_t)blockIdx.x * 256 + threadIdx.x;
    if (i >= MN) return;
    float v = part[i];
    for (int s = 1; s < S; ++s) v += part[s * MN + i];
    y[i] = (uint16_t)(pack_bf16x2(v, 0.f) & 0xFFFF);
}

// Decode GEMM for 32 < M <= 48 and K <= kDecodeKxMaxK: the same per-wave W
// streams of full 128-byte rows, but X stays in LDS for the whole of K and
// the waves split K.  A workgroup owns 96 W rows and all M rows of X; its 8
// waves are 2 column groups of 48 rows (3 subtiles) times 4 K groups, each K
// group a contiguous range of K blocks.  A wave reads the X fragments of a K
// block once and uses them for its 3 subtiles, so an X block is read from LDS
// by 2 waves instead of 6 (with M = 48 the X block is as large as 3 W
// subtiles); the K groups' FP32 partial sums meet in LDS at the end.  (With
// M = 64 and so a 64-row X in LDS, the W ring can hold only two subtile
// stages per wave and the W stream alone takes as long as the 64x96 tile of
// the main kernel: the dispatch keeps that tile there.)
// W comes through a private ring of 3 subtile stages per wave (one subtile of
// one K block, 2 KB, per stage; two stages ahead).  X, its scales and the
// weight scales arrive once, at the start, loaded by all waves together.
constexpr int kDecodeKxMaxK = 1664;
// LDS row stride of an X block kc bytes wide: kc rounded to an odd multiple
// of 128 bytes (with the chunk swizzle, fragment reads of 16 rows then hit
// distinct bank groups).
__host__ __device__ constexpr int decode_stride(int kc) { return (kc & 255) ? kc : kc + 128; }

template <int MSUB>
struct DecodeKxLayout {
    static constexpr int NW = 8, NWN = 2, NWK = 4, SN = 3, NS = 3;
    static constexpr int MR = 16 * MSUB;
    static constexpr int XSTRIDE_MAX = 1664;            // decode_stride(kDecodeKxMaxK)
    static constexpr int KB_MAX = kDecodeKxMaxK / 128;
    static constexpr int X0 = 0;
    static constexpr int SA0 = MR * XSTRIDE_MAX;        // sA [KB][MR] floats
    // (whole 256-byte wave loads: the last one may run past KB*MR floats)
    static constexpr int SB0 = SA0 + (KB_MAX * MR * 4 + 255) / 256 * 256;   // sB [2][KB] floats, one wave load
    static constexpr int W0 = SB0 + 256;                // W rings [wave][stage] 2 KB
    static constexpr int SPARE = W0 + NW * NS * 2048;
    static constexpr int BYTES = SPARE + 1024;
    static constexpr int RED = NW * SN * MSUB * 1024;   // partial sums at the end (over everything)
    static constexpr int LDS = BYTES > RED ? BYTES : RED;
    static_assert(LDS <= 160 * 1024, "LDS");
    static_assert(2 * KB_MAX <= 64, "one wave load holds the sB of two weight blocks");
};

template <int MSUB, bool POW2>
__global__ __launch_bounds__(512, 1) void decode_kx_kernel(
    const uint8_t* __restrict__ xq_, const float* __restrict__ sa_, const uint8_t* __restrict__ wq_,
    const float* __restrict__ sb_, uint16_t* __restrict__ y_, GemmParams p) {
    using L = DecodeKxLayout<MSUB>;
    constexpr int NW = L::NW, NWN = L::NWN, NWK = L::NWK, SN = L::SN, NS = L::NS;
    constexpr int TN = 16 * SN * NWN;
    constexpr int PAIRS = SN * MSUB;
    static_assert(NS == SN, "ring slot = subtile index");
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::LDS];

    const int lane = threadIdx.x & 63;
    const int w = uniform(threadIdx.x >> 6);
    const int wn = w % NWN, wk = w / NWN;
    const int r16 = lane & 15, g = lane >> 4;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int KB = (int)(K >> 7);
    const int xstride = decode_stride((int)K);
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    const int64_t nw = n0 + 16 * SN * wn;              // this wave's first column
    const int kb_lo = wk * KB / NWK, kb_hi = (wk + 1) * KB / NWK;
    const int Q = (kb_hi - kb_lo) * SN;                // this wave's stages: (K block, subtile)
    const uint32_t lds0 = lds_addr(smem);

    const int64_t rows_w = N - n0 < TN ? N - n0 : TN;
    const i32x4 wr = make_rsrc(wq_ + n0 * K, (uint32_t)(rows_w * K));
    const i32x4 xr = make_rsrc(xq_, (uint32_t)(M * K));
    const i32x4 sar = make_rsrc(sa_, (uint32_t)(KB * M * 4));
    const int64_t nb0 = n0 >> 7, nb1 = (n0 + rows_w - 1) >> 7;
    const i32x4 sbr = make_rsrc(sb_ + nb0 * KB, (uint32_t)((nb1 - nb0 + 1) * KB * 4));
    const i32x4 none = make_rsrc(wq_, 0u);
    constexpr uint32_t kFar = 0x7FFFFFF0u;

    // ---- W stage q = (K block kb_lo + q/SN, subtile q%SN), ring slot q%SN ----
    uint32_t wsrc[2];
#pragma unroll
    for (int h = 0; h < 2; ++h) {
        const int r = 8 * h + (lane >> 3);
        wsrc[h] = (uint32_t)((nw - n0 + r) * K) + 16 * ((lane & 7) ^ lds_swz(r));
    }
    const uint32_t wring = lds0 + L::W0 + (uint32_t)w * NS * 2048;
    auto issue_w = [&](int q, auto sc) {               // sc: q % SN as a constant
        constexpr int s = decltype(sc)::value;
        const bool in = q < Q;
        const int kb = kb_lo + q / SN;
        const i32x4 rs = in ? wr : none;
        const uint32_t off = (uint32_t)(16 * s) * (uint32_t)K + (uint32_t)(in ? kb : 0) * 128;
        dma_lds16_one<0>(wring + s * 2048, wsrc[0] + off, rs, 0);
        dma_lds16_one<0>(wring + s * 2048 + 1024, wsrc[1] + off, rs, 0);
    };

    // ---- prologue: W stages 0 and 1, then X, sA, sB (all waves share them) ----
    issue_w(0, std::integral_constant<int, 0>{});
    issue_w(1, std::integral_constant<int, 1>{});
    {
        const int nxl = L::MR * xstride / 1024;         // 1 KB loads of X
        const int nsa = (KB * L::MR * 4 + 255) / 256;   // dword loads of sA
        const int ntot = nxl + nsa + 1;
        for (int i = w; i < ntot; i += NW) {            // wave-uniform
            if (i < nxl) {
                const int d = 1024 * i + 16 * lane;
                const int r = d / xstride, j = (d - r * xstride) >> 4;
                const int c = j ^ lds_swz(r);
                const uint32_t src = (16 * j < K) ? (uint32_t)(r * K + 16 * c) : kFar;
                dma_lds16_one<0>(lds0 + L::X0 + 1024 * i, src, xr, 0);
            } else if (i < nxl + nsa) {
                const int f = 64 * (i - nxl) + lane;    // float f of [KB][MR]
                const int kb = f / L::MR, m = f - kb * L::MR;
                const uint32_t src = (kb < KB && m < M) ? (uint32_t)((kb * M + m) * 4) : kFar;
                dma_lds4(lds0 + L::SA0 + 256 * (i - nxl), src, sar, 0);
            } else {
                // lane b*KB + kb: sB of weight block nb0 + b, K block kb
                const int b = lane / KB, kb = lane - b * KB;
                const uint32_t src = (b < 2) ? (uint32_t)((b * KB + kb) * 4) : kFar;
                dma_lds4(lds0 + L::SB0, src, sbr, 0);
            }
        }
    }
    wait_vmcnt<0>();
    lds_barrier();

    // ---- fragment reads ----
    const int sw = lds_swz(r16);
    const uint32_t wfa = (uint32_t)r16 * 128 + 16 * (g ^ sw), wfb = (uint32_t)r16 * 128 + 16 * ((4 + g) ^ sw);
    const uint32_t xfa = (uint32_t)r16 * xstride + 16 * (g ^ sw);
    const uint32_t xfb = (uint32_t)r16 * xstride + 16 * ((4 + g) ^ sw);
    auto rd16 = [&](uint32_t off) -> i32x4 { return *reinterpret_cast<const i32x4*>(smem + off); };
    int sbl[SN];                                       // weight block of each subtile in the sB table
#pragma unroll
    for (int s = 0; s < SN; ++s) {
        const int64_t ns = nw + 16 * s < N ? nw + 16 * s : N - 1;
        sbl[s] = (int)((ns >> 7) - nb0);
    }
    const float* sbt = reinterpret_cast<const float*>(smem + L::SB0);
    const float* sat = reinterpret_cast<const float*>(smem + L::SA0);

    f32x4 acc[SN][MSUB];
#pragma unroll
    for (int s = 0; s < SN; ++s)
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) acc[s][ms] = f32x4{0.f, 0.f, 0.f, 0.f};

    // ---- K loop: per K block, its SN stages; stage q+2 issued before stage q is used ----
    for (int kb = kb_lo; kb < kb_hi; ++kb) {
        i32x8 xf[MSUB];
        float sav[MSUB];
        const uint32_t xs = L::X0 + 128 * kb;
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) {
            const i32x4 xa = rd16(xs + ms * 16 * xstride + xfa), xb = rd16(xs + ms * 16 * xstride + xfb);
            xf[ms] = i32x8{xa.x, xa.y, xa.z, xa.w, xb.x, xb.y, xb.z, xb.w};
            sav[ms] = sat[kb * L::MR + 16 * ms + r16];
        }
        static_for<SN>([&](auto sc) {
            constexpr int s = decltype(sc)::value;
            const int q = (kb - kb_lo) * SN + s;
            // stage q+2 reuses the ring slot of stage q-1: this wave's reads of
            // it must have completed (the compiler may sink their MFMAs, and
            // with them the wait for the reads, below this point)
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue_w(q + 2, std::integral_constant<int, (s + 2) % SN>{});
            wait_vmcnt<4>();                           // stage q: only stages q+1, q+2 may be in flight
            asm volatile("" ::: "memory");
            const i32x4 wa = rd16(L::W0 + (uint32_t)w * NS * 2048 + s * 2048 + wfa);
            const i32x4 wb = rd16(L::W0 + (uint32_t)w * NS * 2048 + s * 2048 + wfb);
            const i32x8 wf = i32x8{wa.x, wa.y, wa.z, wa.w, wb.x, wb.y, wb.z, wb.w};
            const float sbv = sbt[sbl[s] * KB + kb];
#pragma unroll
            for (int ms = 0; ms < MSUB; ++ms) {
                if constexpr (POW2) {
                    acc[s][ms] = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf, xf[ms], acc[s][ms], 0, 0, 0, e8m0_of(sbv), 0, e8m0_of(sav[ms]));
                } else {
                    const f32x4 part = __builtin_amdgcn_mfma_scale_f32_16x16x128_f8f6f4(
                        wf, xf[ms], f32x4{0.f, 0.f, 0.f, 0.f}, 0, 0, 0, 0, 0, 0);
                    const float sc2 = sav[ms] * sbv;
#pragma unroll
                    for (int r = 0; r < 4; ++r) acc[s][ms][r] = __builtin_fmaf(sc2, part[r], acc[s][ms][r]);
                }
            }
        });
    }
    wait_vmcnt<0>();

    // ---- cross-wave sum in LDS (over everything), then BF16 stores ----
    __syncthreads();
    f32x4* red = reinterpret_cast<f32x4*>(smem);        // [wave][subtile pair][lane]
#pragma unroll
    for (int q = 0; q < PAIRS; ++q) red[(w * PAIRS + q) * 64 + lane] = acc[q / MSUB][q % MSUB];
    __syncthreads();
    for (int t = w; t < NWN * PAIRS; t += NW) {
        const int cg = t / PAIRS, q = t % PAIRS;       // column group, its subtile pair
        f32x4 v = red[(cg * PAIRS + q) * 64 + lane];   // K group 0 (wave cg)
#pragma unroll
        for (int k2 = 1; k2 < NWK; ++k2) {
            const f32x4 u = red[((k2 * NWN + cg) * PAIRS + q) * 64 + lane];
            v = f32x4{v[0] + u[0], v[1] + u[1], v[2] + u[2], v[3] + u[3]};
        }
        const int s = q / MSUB, ms = q % MSUB;
        const int64_t m = 16 * ms + r16;
        const int64_t n = n0 + 16 * SN * cg + 16 * s + 4 * g;
        if (m >= M || n >= N) continue;
        uint16_t* yrow = y_ + m * N;
        const uint32_t lo = pack_bf16x2(v[0], v[1]);
        const uint32_t hi = pack_bf16x2(v[2], v[3]);
        if ((N & 3) == 0 && n + 3 < N) {
            *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
        } else {
            yrow[n] = (uint16_t)(lo & 0xFFFF);
            if (n + 1 < N) yrow[n + 1] = (uint16_t)(lo >> 16);
            if (n + 2 < N) yrow[n + 2] = (uint16_t)(hi & 0xFFFF);
            if (n + 3 < N) yrow[n + 3] = (uint16_t)(hi >> 16);
        }
    }
}

}  // namespace fp8k

namespace fp8k {

// ---------------------------------------------------------------------------
// Exact decode GEMM (M <= 64), the default path for decode-sized M: the
// streaming structure of decode_kernel (per-wave W rings of whole 128-byte
// rows, no barrier per K block; X and scales in chunks shared by the waves),
// with each 128-K block partial formed exactly: E4M3 bytes widened to FP16
// (exact), products by the FP16 matrix instruction (a product of two E4M3
// values has at most 8 significant bits and is exact in its FP32 sum), the
// block partial summed in FP32 and promoted with sA*sB into the FP32
// accumulator (DeepGEMM page, sections "细粒度缩放在 GEMM 层面引爆的两个问题"
// and "主循环骨架": per-block partials in limited precision, promoted into a
// full-precision accumulator).
//   * Wave w owns 32 W rows (output columns) and all rows of X in MSUB 32-row
//     subtiles: 32x32x16 FP16 MFMAs, W the A operand (lane l: column m = l%32
//     of the result, rows n = 8(r/4) + 4(l/32) + r%4 of its 16 values), so a
//     lane holds one sA per subtile and the wave's 32 rows share one sB.
//   * K order inside a block: lane group h = l/32 takes bytes 64h .. 64h+63
//     of its row, step s of the block bytes 64h + 8s .. +7, the same for both
//     operands.
//   * W: 4 KB per K block per wave (four DMAs of 8 whole rows), NS-stage ring,
//     waits on the wave's own vector-memory counter only.
//   * X, sA, sB: chunks of KBC K blocks, double-buffered, issued one chunk
//     ahead by all waves together, one barrier per chunk (as decode_kernel).
//     An X chunk is stored densely (KBC*128 bytes per row, every DMA lane
//     carrying data) with chunk c of row r in slot c ^ (r mod 16): a fragment
//     read of 16 rows at one logical chunk then covers all 64 banks once.
// ---------------------------------------------------------------------------
template <int MSUB, int NW, int NS, int KBC>
struct DecodeExactLayout {
    static constexpr int XSTRIDE = KBC * 128;              // LDS bytes per X row of a chunk
    static constexpr int MR = 32 * MSUB;                   // X rows staged (rows past M read zeros)
    static constexpr int XBYTES = MR * XSTRIDE;
    static constexpr int NXL = XBYTES / 1024;              // 1 KB loads of an X chunk
    static constexpr int NSA = (KBC * MR * 4 + 255) / 256; // dword loads of its sA
    static constexpr int NT = NXL + NSA + 1;               // + one dword load of its sB
    static constexpr int NPW = (NT + NW - 1) / NW;         // chunk loads per wave
    static constexpr int X0 = 0;
    static constexpr int SA0 = 2 * XBYTES;                 // sA [KBC][MR] floats, two buffers
    static constexpr int SB0 = SA0 + 2 * NSA * 256;        // sB [2][KBC] floats, two buffers
    static constexpr int W0 = SB0 + 2 * 256;               // W rings [wave][stage] 4 KB
    static constexpr int SPARE = W0 + NW * NS * 4096;      // target of the surplus chunk loads
    static constexpr int BYTES = SPARE + 1024;
    static_assert(KBC >= 2 && XBYTES % 1024 == 0, "16 chunks per row at least; whole wave loads");
    static_assert(2 * KBC <= 64, "one wave load holds the sB of two weight blocks");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

// Number of multiples of KBC in (q - D, q] for a position q = c*KBC + pos in
// the steady state (c*KBC >= D): the X/scale chunk loads issued between the
// W loads of K block q and its use.
__host__ __device__ constexpr int chunks_between(int pos, int D, int KBC) {
    return D > pos ? (D - pos + KBC - 1) / KBC : 0;
}

template <int MSUB, int NW, int NS, int KBC>
__global__ __launch_bounds__(64 * NW, 1) void decode_exact_kernel(
    const uint8_t* __restrict__ xq_, const float* __restrict__ sa_, const uint8_t* __restrict__ wq_,
    const float* __restrict__ sb_, uint16_t* __restrict__ y_, GemmParams p) {
    using L = DecodeExactLayout<MSUB, NW, NS, KBC>;
    constexpr int D = NS - 1, NPW = L::NPW;
    constexpr int CW = (D + KBC - 1) / KBC;             // chunks before the steady-state waits apply
    static_assert(MSUB >= 1 && MSUB <= 2 && NW >= 1 && NS >= 2, "decode tile");
    static_assert(4 * D + NPW * chunks_between(0, D, KBC) <= 63 && 4 * KBC <= 63, "vmcnt range");
    constexpr int TN = 32 * NW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::BYTES];

    const int lane = threadIdx.x & 63;
    const int w = uniform(threadIdx.x >> 6);
    const int r32 = lane & 31, h = lane >> 5;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int KB = (int)(K >> 7);
    // Split K (grid.y > 1): this workgroup takes the chunks [cs0, cs0 + NC)
    // of the K range and writes FP32 partial sums.
    const int NCT = (KB + KBC - 1) / KBC;
    const int cs0 = (int)(blockIdx.y * NCT / gridDim.y);
    const int NC = (int)((blockIdx.y + 1) * NCT / gridDim.y) - cs0;
    const int kq0 = cs0 * KBC;                          // first K block of this range
    const int NQ = (KB - kq0 < NC * KBC) ? KB - kq0 : NC * KBC;   // K blocks in this range
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    const int64_t nw = n0 + 32 * w;                     // this wave's first column
    const uint32_t lds0 = lds_addr(smem);

    const int64_t rows_w = N - n0 < TN ? N - n0 : TN;
    const i32x4 wr = make_rsrc(wq_ + n0 * K, (uint32_t)(rows_w * K));
    const i32x4 xr = make_rsrc(xq_, (uint32_t)(M * K));
    const i32x4 sar = make_rsrc(sa_, (uint32_t)(KB * M * 4));
    const int64_t nb0 = n0 >> 7, nb1 = (n0 + rows_w - 1) >> 7;
    const i32x4 sbr = make_rsrc(sb_ + nb0 * KB, (uint32_t)((nb1 - nb0 + 1) * KB * 4));
    const i32x4 none = make_rsrc(wq_, 0u);
    constexpr uint32_t kFar = 0x7FFFFFF0u;

    // ---- W: this wave's 32 rows, four 1 KB loads per K block ----
    // load j, lane l: row 8j + l/8, LDS slot l%8 holding chunk (l%8) ^ lds_swz(row)
    uint32_t wsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * j + (lane >> 3);
        wsrc[j] = (uint32_t)((32 * w + r) * K) + 16 * ((lane & 7) ^ lds_swz(r));
    }
    const uint32_t wring = lds0 + L::W0 + (uint32_t)w * NS * 4096;
    auto issue_w = [&](int q) FP8K_INLINE {            // q: position in this range
        const bool in = q < NQ;
        const i32x4 rs = in ? wr : none;
        const uint32_t dst = wring + (uint32_t)(q % NS) * 4096;
        const uint32_t off = (uint32_t)(in ? kq0 + q : 0) * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_lds16_one<0>(dst + 1024 * j, wsrc[j] + off, rs, 0);
    };

    // ---- X, sA, sB of local chunk c: NPW loads per wave, slot i = w + NW*t ----
    auto issue_chunk = [&](int c) FP8K_INLINE {
        const bool in = c < NC;
        const int buf = c & 1;
        const int k0 = (cs0 + c) * KBC * 128, kb0 = (cs0 + c) * KBC;
#pragma unroll
        for (int t = 0; t < NPW; ++t) {
            const int i = w + NW * t;                   // wave-uniform
            if (i < L::NXL) {
                const int d = 1024 * i + 16 * lane;
                const int r = d / L::XSTRIDE, j = (d - r * L::XSTRIDE) >> 4;
                const int cc = j ^ (r & 15);
                dma_lds16_one<0>(lds0 + L::X0 + buf * L::XBYTES + 1024 * i, (uint32_t)(r * K + k0 + 16 * cc),
                                 in ? xr : none, 0);
            } else if (i < L::NXL + L::NSA) {
                const int f = 64 * (i - L::NXL) + lane;      // float f of the chunk's [KBC][MR] sA
                const int kb = f / L::MR, m = f - kb * L::MR;
                const uint32_t src = (in && kb < KBC && m < M) ? (uint32_t)(((kb0 + kb) * M + m) * 4) : kFar;
                dma_lds4(lds0 + L::SA0 + buf * (L::NSA * 256) + 256 * (i - L::NXL), src, in ? sar : none, 0);
            } else if (i < L::NT) {
                // lane b*KBC + kb: sB of weight block nb0 + b, K block kb0 + kb
                const int b = lane / KBC, kb = lane - b * KBC;
                const uint32_t src = (in && b < 2) ? (uint32_t)((b * KB + kb0 + kb) * 4) : kFar;
                dma_lds4(lds0 + L::SB0 + buf * 256, src, in ? sbr : none, 0);
            } else {
                dma_lds16_one<0>(lds0 + L::SPARE, kFar, none, 0);
            }
        }
    };

    // ---- fragments: lane (r32, h) reads logical chunks 4h .. 4h+3 of its row's block ----
    const int sw = lds_swz(r32);
    uint32_t fo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fo[j] = 16u * (uint32_t)((4 * h + j) ^ sw);
    const int sbl = (int)((nw >> 7) - nb0);             // this wave's weight block in the chunk's sB
    auto rd16 = [&](uint32_t off) FP8K_INLINE -> i32x4 { return *reinterpret_cast<const i32x4*>(smem + off); };

    f32x16 acc[MSUB];
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ms][r] = 0.f;

    auto compute = [&](int q, int buf, int kbl) FP8K_INLINE {
        const uint32_t ws = L::W0 + (uint32_t)w * NS * 4096 + (uint32_t)(q % NS) * 4096 + (uint32_t)r32 * 128;
        i32x4 wv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[j] = rd16(ws + fo[j]);
        // X row 32 ms + r32, logical chunk 8 kbl + 4h + j in slot (8 kbl + 4h + j) ^ (r32 mod 16)
        const uint32_t xs = L::X0 + buf * L::XBYTES + (uint32_t)r32 * L::XSTRIDE;
        i32x4 xv[MSUB][4];
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
            for (int j = 0; j < 4; ++j)
                xv[ms][j] = rd16(xs + 32 * ms * L::XSTRIDE + 16 * ((8 * kbl + 4 * h + j) ^ (r32 & 15)));
        const float sbv = *reinterpret_cast<const float*>(smem + L::SB0 + buf * 256 + 4 * (sbl * KBC + kbl));
        const float* sap = reinterpret_cast<const float*>(smem + L::SA0 + buf * (L::NSA * 256)) + kbl * L::MR + r32;
        f32x16 part[MSUB];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int j = s >> 1, o = 2 * (s & 1);
            const f16x8 a = e4m3x8_to_f16(wv[j][o], wv[j][o + 1]);
#pragma unroll
            for (int ms = 0; ms < MSUB; ++ms) {
                const f16x8 b = e4m3x8_to_f16(xv[ms][j][o], xv[ms][j][o + 1]);
                part[ms] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, s == 0 ? f32x16{} : part[ms], 0, 0, 0);
            }
        }
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) {
            const float f = sap[32 * ms] * sbv;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ms][r] = __builtin_fmaf(f, part[ms][r], acc[ms][r]);
        }
    };

    // ---- issue order and waits ----
    // Position q (K block kq0 + q) of local chunk c = q / KBC: at the start of
    // a chunk the wave waits for that chunk (issued one chunk earlier, before
    // the KBC W blocks of the previous chunk: 4*KBC loads after it; chunk 0:
    // the 4*D prologue W loads), a barrier publishes it and frees the other
    // buffer, and the next chunk is issued.  Before K block q is used, the W
    // blocks q+1 .. q+D (4 loads each) and the chunks issued at positions in
    // (q-D, q] may still be in flight.  In the first CW chunks fewer chunk
    // loads than that follow W block q, so the wait there counts W loads only
    // (a stricter wait).
    issue_chunk(0);
#pragma unroll
    for (int j = 0; j < D; ++j) issue_w(j);
    for (int c = 0; c < NC; ++c) {
        if (c == 0) wait_vmcnt<4 * D>();
        else wait_vmcnt<4 * KBC>();
        asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");
        issue_chunk(c + 1);
        const bool steady = c >= CW;
        static_for<KBC>([&](auto pc) FP8K_INLINE {
            constexpr int pos = decltype(pc)::value;
            const int q = c * KBC + pos;
            // position q+D reuses the ring slot of position q-1: this wave's
            // reads of it must have completed
            asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
            issue_w(q + D);
            if (steady) wait_vmcnt<4 * D + NPW * chunks_between(pos, D, KBC)>();
            else wait_vmcnt<4 * D>();
            asm volatile("" ::: "memory");
            if (q < NQ) compute(q, c & 1, pos);
        });
    }
    wait_vmcnt<0>();

    // ---- stores: lane holds m = 32 ms + r32, n = nw + 8k + 4h + (0..3), k = 0..3 ----
    float* part_base = p.part ? p.part + (int64_t)blockIdx.y * M * N : nullptr;
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms) {
        const int64_t m = 32 * ms + r32;
        if (m >= M) continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t n = nw + 8 * k + 4 * h;
            if (n >= N) continue;
            if (part_base) {
                float* prow = part_base + m * N;
                if ((N & 3) == 0 && n + 3 < N) {
                    *reinterpret_cast<f32x4*>(prow + n) =
                        f32x4{acc[ms][4 * k], acc[ms][4 * k + 1], acc[ms][4 * k + 2], acc[ms][4 * k + 3]};
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) prow[n + r] = acc[ms][4 * k + r];
                }
                continue;
            }
            uint16_t* yrow = y_ + m * N;
            const uint32_t lo = pack_bf16x2(acc[ms][4 * k], acc[ms][4 * k + 1]);
            const uint32_t hi = pack_bf16x2(acc[ms][4 * k + 2], acc[ms][4 * k + 3]);
            if ((N & 3) == 0 && n + 3 < N) {
                *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
            } else {
                yrow[n] = (uint16_t)(lo & 0xFFFF);
                if (n + 1 < N) yrow[n + 1] = (uint16_t)(lo >> 16);
                if (n + 2 < N) yrow[n + 2] = (uint16_t)(hi & 0xFFFF);
                if (n + 3 < N) yrow[n + 3] = (uint16_t)(hi >> 16);
            }
        }
    }
}

}  // namespace fp8k

namespace fp8k {

// ---------------------------------------------------------------------------
// Exact decode GEMM with X resident in LDS (M <= 64, a K range of at most
// KBMAX blocks per workgroup): the same exact block partials and per-wave W
// rings as decode_exact_kernel, but X, its scales and the weight scales of
// the workgroup's K range are loaded once, before the K loop, so that the
// loop holds no barrier and no chunk loads: per K block a wave issues the
// four W loads D blocks ahead, waits for the block in hand and computes it.
//   * Every workgroup reads the same X: each starts its X loads at a
//     different 1 KB piece (rotated by its index), so that the workgroups of
//     an XCD do not all ask the same L2 channel for the same lines at once.
//   * X rows in LDS: stride XS = the range's bytes rounded to an odd multiple
//     of 128, chunk c of a K block at slot c ^ lds_swz(row) inside its block
//     (fragment reads of 16 rows at one logical chunk then hit distinct bank
//     groups).
//   * Split K (grid.y > 1): workgroup (t, s) takes K blocks
//     [s*KB/S, (s+1)*KB/S) and writes FP32 partial sums [s][M][N].
// ---------------------------------------------------------------------------
template <int MSUB, int NW, int NS, int KBMAX>
struct DecodeExactXLayout {
    static constexpr int MR = 32 * MSUB;
    static constexpr int XS_MAX = decode_stride(KBMAX * 128);
    static constexpr int X0 = 0;
    static constexpr int XBYTES = MR * XS_MAX;
    static constexpr int SA0 = (XBYTES + 1023) / 1024 * 1024;  // sA [KBr][MR] floats
    static constexpr int SA_BYTES = (KBMAX * MR * 4 + 255) / 256 * 256;
    static constexpr int SB0 = SA0 + SA_BYTES;                 // sB [2][KBr] floats, one wave load
    static constexpr int W0 = SB0 + 256;                       // W rings [wave][stage] 4 KB
    static constexpr int BYTES = W0 + NW * NS * 4096;
    static_assert(2 * KBMAX <= 64, "one wave load holds the sB of two weight blocks");
    static_assert(BYTES <= 160 * 1024, "LDS");
};

template <int MSUB, int NW, int NS, int KBMAX>
__global__ __launch_bounds__(64 * NW, 1) void decode_exact_x_kernel(
    const uint8_t* __restrict__ xq_, const float* __restrict__ sa_, const uint8_t* __restrict__ wq_,
    const float* __restrict__ sb_, uint16_t* __restrict__ y_, GemmParams p) {
    using L = DecodeExactXLayout<MSUB, NW, NS, KBMAX>;
    constexpr int D = NS - 1;
    static_assert(MSUB >= 1 && MSUB <= 2 && NW >= 1 && NS >= 2 && 4 * D <= 63, "decode tile");
    constexpr int TN = 32 * NW;
    __shared__ __attribute__((aligned(1024))) uint8_t smem[L::BYTES];

    const int lane = threadIdx.x & 63;
    const int w = uniform(threadIdx.x >> 6);
    const int r32 = lane & 31, h = lane >> 5;
    const int64_t M = p.M, N = p.N, K = p.K;
    const int KB = (int)(K >> 7);
    const int kb0 = (int)(blockIdx.y * KB / gridDim.y);
    const int NQ = (int)((blockIdx.y + 1) * KB / gridDim.y) - kb0;   // K blocks of this range (<= KBMAX)
    const int xs = decode_stride(NQ * 128);              // LDS row stride of X
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    const int64_t nw = n0 + 32 * w;
    const uint32_t lds0 = lds_addr(smem);

    const int64_t rows_w = N - n0 < TN ? N - n0 : TN;
    const i32x4 wr = make_rsrc(wq_ + n0 * K, (uint32_t)(rows_w * K));
    const i32x4 xr = make_rsrc(xq_, (uint32_t)(M * K));
    const i32x4 sar = make_rsrc(sa_, (uint32_t)(KB * M * 4));
    const int64_t nb0 = n0 >> 7, nb1 = (n0 + rows_w - 1) >> 7;
    const i32x4 sbr = make_rsrc(sb_ + nb0 * KB, (uint32_t)((nb1 - nb0 + 1) * KB * 4));
    const i32x4 none = make_rsrc(wq_, 0u);
    constexpr uint32_t kFar = 0x7FFFFFF0u;

    // ---- prologue: X rows [0, MR) x K blocks [kb0, kb0 + NQ), sA, sB (all waves) ----
    {
        const int nxl = L::MR * xs / 1024;               // whole 1 KB loads (MR*xs is a multiple of 1 KB)
        const int nsa = (NQ * L::MR * 4 + 255) / 256;
        const int ntot = nxl + nsa + 1;
        const int rot = (int)(blockIdx.x % (unsigned)nxl);
        for (int i = w; i < ntot; i += NW) {             // wave-uniform
            if (i < nxl) {
                const int ir = i + rot < nxl ? i + rot : i + rot - nxl;   // rotated 1 KB piece
                const int d = 1024 * ir + 16 * lane;
                const int r = d / xs, j = (d - r * xs) >> 4;
                const int c = (j & ~7) | ((j & 7) ^ lds_swz(r));   // logical chunk in slot j
                const uint32_t src = (16 * j < NQ * 128) ? (uint32_t)(r * K + kb0 * 128 + 16 * c) : kFar;
                dma_lds16_one<0>(lds0 + L::X0 + 1024 * ir, src, xr, 0);
            } else if (i < nxl + nsa) {
                const int f = 64 * (i - nxl) + lane;     // float f of [NQ][MR]
                const int kb = f / L::MR, m = f - kb * L::MR;
                const uint32_t src = (kb < NQ && m < M) ? (uint32_t)(((kb0 + kb) * M + m) * 4) : kFar;
                dma_lds4(lds0 + L::SA0 + 256 * (i - nxl), src, sar, 0);
            } else {
                // lane b*NQ + kb: sB of weight block nb0 + b, K block kb0 + kb
                const int b = lane / NQ, kb = lane - b * NQ;
                const uint32_t src = (b < 2) ? (uint32_t)((b * KB + kb0 + kb) * 4) : kFar;
                dma_lds4(lds0 + L::SB0, src, sbr, 0);
            }
        }
    }

    // ---- W: this wave's 32 rows, four 1 KB loads per K block ----
    // load j, lane l: row 8j + l/8, LDS slot l%8 holding chunk (l%8) ^ lds_swz(row)
    uint32_t wsrc[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) {
        const int r = 8 * j + (lane >> 3);
        wsrc[j] = (uint32_t)((32 * w + r) * K) + 16 * ((lane & 7) ^ lds_swz(r));
    }
    const uint32_t wring = lds0 + L::W0 + (uint32_t)w * NS * 4096;
    auto issue_w = [&](int q) FP8K_INLINE {
        const bool in = q < NQ;
        const i32x4 rs = in ? wr : none;
        const uint32_t dst = wring + (uint32_t)(q % NS) * 4096;
        const uint32_t off = (uint32_t)(in ? kb0 + q : 0) * 128;
#pragma unroll
        for (int j = 0; j < 4; ++j) dma_lds16_one<0>(dst + 1024 * j, wsrc[j] + off, rs, 0);
    };
#pragma unroll
    for (int j = 0; j < D; ++j) issue_w(j);
    // this wave's prologue loads are the ones before the 4*D W loads
    wait_vmcnt<4 * D>();
    asm volatile("s_waitcnt lgkmcnt(0)\n\ts_barrier" ::: "memory");

    const int sw = lds_swz(r32);
    uint32_t fo[4];
#pragma unroll
    for (int j = 0; j < 4; ++j) fo[j] = 16u * (uint32_t)((4 * h + j) ^ sw);
    const int sbl = (int)((nw >> 7) - nb0);
    const float* sat = reinterpret_cast<const float*>(smem + L::SA0);
    const float* sbt = reinterpret_cast<const float*>(smem + L::SB0);
    auto rd16 = [&](uint32_t off) FP8K_INLINE -> i32x4 { return *reinterpret_cast<const i32x4*>(smem + off); };

    f32x16 acc[MSUB];
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
        for (int r = 0; r < 16; ++r) acc[ms][r] = 0.f;

    for (int q = 0; q < NQ; ++q) {
        // block q+D reuses the ring slot of block q-1: its reads have completed
        asm volatile("s_waitcnt lgkmcnt(0)" ::: "memory");
        issue_w(q + D);
        wait_vmcnt<4 * D>();
        asm volatile("" ::: "memory");
        const uint32_t wsl = L::W0 + (uint32_t)w * NS * 4096 + (uint32_t)(q % NS) * 4096 + (uint32_t)r32 * 128;
        i32x4 wv[4];
#pragma unroll
        for (int j = 0; j < 4; ++j) wv[j] = rd16(wsl + fo[j]);
        const uint32_t xrow = L::X0 + (uint32_t)r32 * xs + 128 * q;
        i32x4 xv[MSUB][4];
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms)
#pragma unroll
            for (int j = 0; j < 4; ++j) xv[ms][j] = rd16(xrow + 32 * ms * xs + fo[j]);
        const float sbv = sbt[sbl * NQ + q];
        f32x16 part[MSUB];
#pragma unroll
        for (int s = 0; s < 8; ++s) {
            const int j = s >> 1, o = 2 * (s & 1);
            const f16x8 a = e4m3x8_to_f16(wv[j][o], wv[j][o + 1]);
#pragma unroll
            for (int ms = 0; ms < MSUB; ++ms) {
                const f16x8 b = e4m3x8_to_f16(xv[ms][j][o], xv[ms][j][o + 1]);
                part[ms] = __builtin_amdgcn_mfma_f32_32x32x16_f16(a, b, s == 0 ? f32x16{} : part[ms], 0, 0, 0);
            }
        }
#pragma unroll
        for (int ms = 0; ms < MSUB; ++ms) {
            const float f = sat[q * L::MR + 32 * ms + r32] * sbv;
#pragma unroll
            for (int r = 0; r < 16; ++r) acc[ms][r] = __builtin_fmaf(f, part[ms][r], acc[ms][r]);
        }
    }
    wait_vmcnt<0>();

    // ---- stores: lane holds m = 32 ms + r32, n = nw + 8k + 4h + (0..3), k = 0..3 ----
    float* part_base = p.part ? p.part + (int64_t)blockIdx.y * M * N : nullptr;
#pragma unroll
    for (int ms = 0; ms < MSUB; ++ms) {
        const int64_t m = 32 * ms + r32;
        if (m >= M) continue;
#pragma unroll
        for (int k = 0; k < 4; ++k) {
            const int64_t n = nw + 8 * k + 4 * h;
            if (n >= N) continue;
            if (part_base) {
                float* prow = part_base + m * N;
                if ((N & 3) == 0 && n + 3 < N) {
                    *reinterpret_cast<f32x4*>(prow + n) =
                        f32x4{acc[ms][4 * k], acc[ms][4 * k + 1], acc[ms][4 * k + 2], acc[ms][4 * k + 3]};
                } else {
#pragma unroll
                    for (int r = 0; r < 4; ++r)
                        if (n + r < N) prow[n + r] = acc[ms][4 * k + r];
                }
                continue;
            }
            uint16_t* yrow = y_ + m * N;
            const uint32_t lo = pack_bf16x2(acc[ms][4 * k], acc[ms][4 * k + 1]);
            const uint32_t hi = pack_bf16x2(acc[ms][4 * k + 2], acc[ms][4 * k + 3]);
            if ((N & 3) == 0 && n + 3 < N) {
                *reinterpret_cast<uint2*>(yrow + n) = make_uint2(lo, hi);
            } else {
                yrow[n] = (uint16_t)(lo & 0xFFFF);
                if (n + 1 < N) yrow[n + 1] = (uint16_t)(lo >> 16);
                if (n + 2 < N) yrow[n + 2] = (uint16_t)(hi & 0xFFFF);
                if (n + 3 < N) yrow[n + 3] = (uint16_t)(hi >> 16);
            }
        }
    }
}

}  // namespace fp8k
