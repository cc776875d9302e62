// kernels_quant.h -- fine-grained E4M3 quantizers for gfx950.
//
// DeepGEMM page ("DeepGEMM 完全拆解"), section "离群值如何摧毁 per-tensor 量化":
// activations take one scale per 1x128 tile (one token, 128 channels),
// weights one scale per 128x128 block; each scale maps the group's absolute
// maximum onto the E4M3 limit 448 and is computed online from the group.
//
// Both kernels are HBM streams: FP32 in (4 B/element), codes out
// (1 B/element) plus one FP32 scale per group.  Loads are 16 B per lane and
// fully coalesced; the group maximum is reduced with cross-lane shuffles.
// The codes are the E4M3 rounding of the correctly rounded FP32 quotient
// x / s, obtained from the product with the rounded reciprocal where that
// provably gives the same code and from an IEEE division elsewhere
// (cvt_e4m3x4_quot).
#pragma once

#include "device_common.h"

namespace fp8k {

// Half-wave (32 lanes) reduction of a maximum.
__device__ __forceinline__ float halfwave_max(float v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 32));
    return v;
}

// Streaming loads: the FP32 inputs are read once, so their loads carry the
// nontemporal hint and do not allocate in the caches.  That matters when the
// caches hold dirty lines of earlier kernels, whose write-back an allocating
// load would wait for (measured after a kernel that left the caches dirty:
// 2.7 -> 4.8 TB/s for the 1x128 quantizer, 2.7 -> 5.4 TB/s for the 128x128
// one; within a few percent on clean caches).  The codes are stored normally:
// the GEMM that follows reads them, and finds them cached (nontemporal code
// stores measured slower over the quantize + GEMM step).
__device__ __forceinline__ f32x4 load_stream(const float* p) {
    return __builtin_nontemporal_load(reinterpret_cast<const f32x4*>(p));
}
__device__ __forceinline__ void store_codes(uint8_t* p, uint32_t v) {
    *reinterpret_cast<uint32_t*>(p) = v;
}
__device__ __forceinline__ float abs_max4(f32x4 v) {
    return fmaxf(fmaxf(fabsf(v[0]), fabsf(v[1])), fmaxf(fabsf(v[2]), fabsf(v[3])));
}

// E4M3 codes of the correctly rounded quotients v[i] / s, with r the
// correctly rounded 1 / s.  The product v[i] * r carries two roundings of
// relative error at most 2^-24 each, so it lies within 2 units in the last
// place of the exact quotient and within 2.5 of the correctly rounded one
// (5 units of the lower binade where the two straddle a power of two).  The
// conversion to E4M3 (round to nearest even, saturating) is monotone in the
// magnitude: when the magnitudes 8 units below and 8 above the product take
// the same code, every value between them does, the correctly rounded
// quotient included, and the product's code (its sign is the quotient's) is
// the answer.  Otherwise -- a product within 8 units of a rounding boundary,
// about 2e-5 of random inputs -- the four quotients are divided.  With a
// power-of-two scale the product is the quotient itself.
template <bool POW2>
__device__ __forceinline__ uint32_t cvt_e4m3x4_quot(f32x4 v, float s, float r) {
    const float q0 = v[0] * r, q1 = v[1] * r, q2 = v[2] * r, q3 = v[3] * r;
    if constexpr (POW2) {
        return cvt_e4m3x4(q0, q1, q2, q3);
    } else {
        const uint32_t a0 = __float_as_uint(q0) & 0x7FFFFFFFu, a1 = __float_as_uint(q1) & 0x7FFFFFFFu;
        const uint32_t a2 = __float_as_uint(q2) & 0x7FFFFFFFu, a3 = __float_as_uint(q3) & 0x7FFFFFFFu;
        auto below = [](uint32_t a) { return __uint_as_float(a > 8u ? a - 8u : 0u); };
        auto above = [](uint32_t a) { return __uint_as_float(a + 8u); };
        const uint32_t lo = cvt_e4m3x4(below(a0), below(a1), below(a2), below(a3));
        const uint32_t hi = cvt_e4m3x4(above(a0), above(a1), above(a2), above(a3));
        if (lo == hi) return cvt_e4m3x4(q0, q1, q2, q3);
        return cvt_e4m3x4(v[0] / s, v[1] / s, v[2] / s, v[3] / s);
    }
}

// 1x128 activation quantizer.  A wave takes one row and up to 8 consecutive
// groups of it (4 KB of FP32): lane l loads 16 bytes of each of 4 row
// segments of 256 values, so each wave load covers 1 KB contiguous and holds
// two groups (one per half-wave); all 4 loads are issued before the first
// reduction.  A 256-thread block takes 4 such units.  Only a row's last unit
// can be short (K/128 not a multiple of 8): it takes the predicated path.
//   x (M,K) fp32 -> xq (M,K) u8, sa [K/128][M] fp32
template <bool POW2, bool PARTIAL>
__device__ __forceinline__ void quant_1x128_unit(const float* __restrict__ x, uint8_t* __restrict__ xq,
                                                 float* __restrict__ sa, int64_t M, int64_t K,
                                                 int64_t KB, int64_t m, int64_t kb0, int lane) {
    const int half = lane >> 5;
    const int64_t off = m * K + kb0 * 128 + lane * 4;
    f32x4 v[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        // group kb0 + 2q + half; groups past the row end are not read
        if (!PARTIAL || kb0 + 2 * q + half < KB) v[q] = load_stream(x + off + 256 * q);
        else v[q] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
    float sg[4];
#pragma unroll
    for (int q = 0; q < 4; ++q) {
        const int64_t kb = kb0 + 2 * q + half;
        const float amax = halfwave_max(abs_max4(v[q]));
        const float s = group_scale(amax, POW2);
        sg[q] = s;
        if (!PARTIAL || kb < KB) store_codes(xq + off + 256 * q, cvt_e4m3x4_quot<POW2>(v[q], s, 1.0f / s));
    }
    // the unit's 8 scales from lanes 0..7 in one store: lane i < 8 takes the
    // scale of group kb0 + i, held by every lane of half i % 2 as sg[i / 2]
    const int i8 = lane & 7;
    const float mine = i8 < 2 ? sg[0] : i8 < 4 ? sg[1] : i8 < 6 ? sg[2] : sg[3];
    const float sc = __shfl(mine, ((lane & 1) << 5) | i8);
    if (lane < 8 && (!PARTIAL || kb0 + lane < KB)) sa[(kb0 + lane) * M + m] = sc;
}

template <bool POW2>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const float* __restrict__ x,
                                                          uint8_t* __restrict__ xq,
                                                          float* __restrict__ sa, int64_t M,
                                                          int64_t K, int64_t units) {
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= units) return;
    const int lane = threadIdx.x & 63;
    const int64_t KB = K / 128;
    const int64_t upr = (KB + 7) / 8;   // units per row
    const int64_t m = u / upr;
    const int64_t kb0 = (u - m * upr) * 8;
    if (kb0 + 8 <= KB) quant_1x128_unit<POW2, false>(x, xq, sa, M, K, KB, m, kb0, lane);
    else quant_1x128_unit<POW2, true>(x, xq, sa, M, K, KB, m, kb0, lane);
}

// 128x128 weight quantizer.  One 256-thread block per (nb, kb) block: thread
// t owns column chunk t%32 (4 floats) of rows t/32, t/32+8, ..., so each
// wave-row load covers 512 contiguous bytes.  The 64 values stay in
// registers between the max pass and the encode pass.  Only the last block
// row can be short (N not a multiple of 128): it takes the predicated path.
//   w (N,K) fp32 -> wq (N,K) u8, sb [ceil(N/128)][K/128] fp32
template <bool POW2, bool PARTIAL>
__device__ __forceinline__ void quant_128x128_block(const float* __restrict__ w, uint8_t* __restrict__ wq,
                                                    float* __restrict__ sb, int64_t N, int64_t K,
                                                    int64_t nb, int64_t kb, float* wave_max) {
    const int64_t KB = K / 128;
    const int c = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const int64_t n0 = nb * 128;
    const int64_t off = (n0 + r0) * K + kb * 128 + c * 4;   // row r0 of the block
    const int64_t rstep = 8 * K;                             // 8 rows further
    f32x4 v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (!PARTIAL || n0 + r0 + 8 * i < N) {
            v[i] = load_stream(w + off + rstep * i);
            amax = fmaxf(amax, abs_max4(v[i]));
        } else {
            v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
        }
    }
#pragma unroll
    for (int o = 32; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 64));
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    const float s = group_scale(amax, POW2);
    const float r = 1.0f / s;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        if (!PARTIAL || n0 + r0 + 8 * i < N) store_codes(wq + off + rstep * i, cvt_e4m3x4_quot<POW2>(v[i], s, r));
    }
    if (threadIdx.x == 0) sb[nb * KB + kb] = s;
}

template <bool POW2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const float* __restrict__ w,
                                                            uint8_t* __restrict__ wq,
                                                            float* __restrict__ sb, int64_t N,
                                                            int64_t K) {
    __shared__ float wave_max[4];
    const int64_t KB = K / 128;
    const int64_t nb = blockIdx.x / KB, kb = blockIdx.x - nb * KB;
    if ((nb + 1) * 128 <= N) quant_128x128_block<POW2, false>(w, wq, sb, N, K, nb, kb, wave_max);
    else quant_128x128_block<POW2, true>(w, wq, sb, N, K, nb, kb, wave_max);
}

// MXFP8 quantizer, for activations and weights alike: one E8M0 scale per 1x32
// group along K (tcgen05 page, sections 6.1 and 6.3: MX formats share one
// power-of-two scale over 32 elements).  The scale is the power of two at or
// above max(amax, 1e-4)/448 (the UE8M0 rule of the 1x128 groups), so no code
// saturates.  A wave takes one row and up to 32 consecutive groups (4 KB of
// FP32): lane l loads 16 bytes of each of 4 row segments of 256 values, so
// eight neighbouring lanes hold one group and its maximum is an 8-lane
// reduction.  Only a row's last unit can be short (K/128 not a multiple of 8).
// The scale bytes are packed 4 to a dword per (K block, row) and the dwords
// laid out [K/128][R] -- DeepGEMM's Blackwell path, tcgen05 page section 5.4,
// takes packed, transposed UE8M0 scales -- so that a GEMM tile reads the
// scales of one K block for consecutive rows from consecutive dwords.
//   x (R, K) fp32 -> q (R, K) u8, e u32 [K/128][R]: byte t of e[kb][r] is the
//   scale byte of group 4kb+t of row r (the scale is 2^(byte-127))
template <bool PARTIAL>
__device__ __forceinline__ void quant_mx_unit(const float* __restrict__ x, uint8_t* __restrict__ q,
                                              uint8_t* __restrict__ e, int64_t R, int64_t K, int64_t G,
                                              int64_t r, int64_t g0, int lane) {
    const int64_t off = r * K + g0 * 32 + lane * 4;
    f32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        // group g0 + 8i + lane/8; groups past the row end are not read
        if (!PARTIAL || g0 + 8 * i + (lane >> 3) < G) v[i] = load_stream(x + off + 256 * i);
        else v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t grp = g0 + 8 * i + (lane >> 3);
        float amax = abs_max4(v[i]);
#pragma unroll
        for (int o = 4; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 8));
        const float s = group_scale(amax, true);
        // s is a power of two: 1/s is exact, and so is x * (1/s) = x / s
        const float inv = 1.0f / s;
        if (!PARTIAL || grp < G) {
            store_codes(q + off + 256 * i, cvt_e4m3x4(v[i][0] * inv, v[i][1] * inv, v[i][2] * inv, v[i][3] * inv));
            if ((lane & 7) == 0) e[((grp >> 2) * R + r) * 4 + (grp & 3)] = (uint8_t)(__float_as_uint(s) >> 23);
        }
    }
}

__global__ __launch_bounds__(256) void quant_mx_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                       uint8_t* __restrict__ e, int64_t R, int64_t K,
                                                       int64_t units) {
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= units) return;
    const int lane = threadIdx.x & 63;
    const int64_t G = K / 32;
    const int64_t upr = (G + 31) / 32;   // units per row
    const int64_t r = u / upr;
    const int64_t g0 = (u - r * upr) * 32;
    if (g0 + 32 <= G) quant_mx_unit<false>(x, q, e, R, K, G, r, g0, lane);
    else quant_mx_unit<true>(x, q, e, R, K, G, r, g0, lane);
}

// Two binary32 values to a byte of two E2M1 nibbles (the first one low) with
// the hardware converter at scale 1: round to nearest, ties to the even code,
// the sign kept -- checked bit-exact against the reference encoder on every
// E2M1 midpoint and its neighbours, both signs.  (E2M1 magnitudes: 0, 0.5, 1,
// 1.5, 2, 3, 4, 6 for codes 0..7.)  sel picks the byte of `old` written.
__device__ __forceinline__ uint32_t cvt_e2m1x2(uint32_t old, float a, float b, int sel) {
    return sel == 0 ? __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 0)
                    : __builtin_amdgcn_cvt_scalef32_pk_fp4_f32(old, a, b, 1.0f, 1);
}

// MXFP4 quantizer for weights: E2M1 elements with one E8M0 scale per 1x32
// group along K (tcgen05 page, section 6.3), the scale being the power of two
// at or above max(amax, 1e-4)/6 (6 = the largest E2M1 magnitude), so no
// element saturates.  Elements are packed two per byte along K, the even one
// in the low nibble.  Same wave units as the MXFP8 quantizer: one row and up
// to 32 groups per wave, 8 lanes per group; each lane packs its 4 values into
// 2 bytes.  The scale bytes go into the packed [K/128][R] dwords.
//   x (R, K) fp32 -> q (R, K/2) u8, e u32 [K/128][R]
template <bool PARTIAL>
__device__ __forceinline__ void quant_mxfp4_unit(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                 uint8_t* __restrict__ e, int64_t R, int64_t K, int64_t G,
                                                 int64_t r, int64_t g0, int lane) {
    const int64_t off = r * K + g0 * 32 + lane * 4;
    f32x4 v[4];
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        if (!PARTIAL || g0 + 8 * i + (lane >> 3) < G) v[i] = load_stream(x + off + 256 * i);
        else v[i] = f32x4{0.f, 0.f, 0.f, 0.f};
    }
#pragma unroll
    for (int i = 0; i < 4; ++i) {
        const int64_t grp = g0 + 8 * i + (lane >> 3);
        float amax = abs_max4(v[i]);
#pragma unroll
        for (int o = 4; o >= 1; o >>= 1) amax = fmaxf(amax, __shfl_xor(amax, o, 8));
        const float a = amax > 1e-4f ? amax : 1e-4f;
        uint32_t bits = __float_as_uint(a / 6.0f);
        if (bits & 0x007FFFFFu) bits = ((bits >> 23) + 1u) << 23;
        // a power of two: 1/s is exact, and so is x * (1/s) = x / s
        const float inv = 1.0f / __uint_as_float(bits);
        if (!PARTIAL || grp < G) {
            const uint32_t p = cvt_e2m1x2(cvt_e2m1x2(0u, v[i][0] * inv, v[i][1] * inv, 0),
                                          v[i][2] * inv, v[i][3] * inv, 1);
            *reinterpret_cast<uint16_t*>(q + off / 2 + 128 * i) = (uint16_t)p;
            if ((lane & 7) == 0) e[((grp >> 2) * R + r) * 4 + (grp & 3)] = (uint8_t)(bits >> 23);
        }
    }
}

__global__ __launch_bounds__(256) void quant_mxfp4_kernel(const float* __restrict__ x, uint8_t* __restrict__ q,
                                                          uint8_t* __restrict__ e, int64_t R, int64_t K,
                                                          int64_t units) {
    const int64_t u = (int64_t)blockIdx.x * 4 + (threadIdx.x >> 6);
    if (u >= units) return;
    const int lane = threadIdx.x & 63;
    const int64_t G = K / 32;
    const int64_t upr = (G + 31) / 32;
    const int64_t r = u / upr;
    const int64_t g0 = (u - r * upr) * 32;
    if (g0 + 32 <= G) quant_mxfp4_unit<false>(x, q, e, R, K, G, r, g0, lane);
    else quant_mxfp4_unit<true>(x, q, e, R, K, G, r, g0, lane);
}

}  // namespace fp8k
