// kernels_decode.h -- block-scaled E4M3 NT GEMM for decode-sized M (M <= 64)
// on gfx950.
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
    const int NC = (KB + KBC - 1) / KBC;
    const int64_t n0 = (int64_t)blockIdx.x * TN;
    // Workgroups walk the K chunks in rotated orders (sequence chunk c is data
    // chunk (c + rot) mod NC), so that at any moment they read different parts
    // of X rather than all the same lines.
    const int rot = (int)(blockIdx.x % (unsigned)NC);
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
        const int cd = c + rot < NC ? c + rot : c + rot - NC;
        return cd * KBC + (q - c * KBC);
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
        const int cd = c + rot < NC ? c + rot : c + rot - NC;   // data chunk
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
        lds_barrier();                                 // chunk c published, buffer of chunk c-1 free
        issue_chunk(c + 1);
        static_for<KBC>([&](auto pc) {
            constexpr int pos = decltype(pc)::value;
            const int q = c * KBC + pos;               // sequence position
            // position q+D reuses the ring slot of position q-1: its reads stay above
            asm volatile("" ::: "memory");
            issue_w(q + D);
            // loads issued after position q's W block: the next D W blocks,
            // and chunk c+1 when position q's block was issued before it
            wait_vmcnt<2 * D + (pos < D ? NPW : 0)>();
            asm volatile("" ::: "memory");
            if (seq_kb(q) < KB) compute(q, c & 1, pos);
        });
    }
    wait_vmcnt<0>();

    // ---- BF16 stores: lane holds n = nw + 4g + r, m = 16 ms + r16 ----
    const int64_t n = nw + 4 * g;
    if (n < N) {
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
