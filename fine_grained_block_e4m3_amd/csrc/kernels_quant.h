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
#pragma once

#include "device_common.h"

namespace fp8k {

// Half-wave (32 lanes) reduction of a maximum.
__device__ __forceinline__ float halfwave_max(float v) {
#pragma unroll
    for (int off = 16; off >= 1; off >>= 1) v = fmaxf(v, __shfl_xor(v, off, 32));
    return v;
}

// 1x128 activation quantizer.  One half-wave per group; a 256-thread block
// handles 8 groups with consecutive m and the same kb, so the 8 scales it
// writes to sa[kb][m..m+7] are contiguous.
//   x (M,K) fp32 -> xq (M,K) u8, sa [K/128][M] fp32
template <bool POW2>
__global__ __launch_bounds__(256) void quant_1x128_kernel(const float* __restrict__ x,
                                                          uint8_t* __restrict__ xq,
                                                          float* __restrict__ sa, int64_t M,
                                                          int64_t K, int64_t groups) {
    const int64_t g = (int64_t)blockIdx.x * 8 + (threadIdx.x >> 5);
    if (g >= groups) return;
    const int lane = threadIdx.x & 31;
    const int64_t kb = g / M, m = g - kb * M;
    const int64_t off = m * K + kb * 128 + lane * 4;
    const float4 v = *reinterpret_cast<const float4*>(x + off);
    float amax = fmaxf(fmaxf(fabsf(v.x), fabsf(v.y)), fmaxf(fabsf(v.z), fabsf(v.w)));
    amax = halfwave_max(amax);
    const float s = group_scale(amax, POW2);
    const uint32_t q = cvt_e4m3x4(v.x / s, v.y / s, v.z / s, v.w / s);
    *reinterpret_cast<uint32_t*>(xq + off) = q;
    if (lane == 0) sa[kb * M + m] = s;
}

// 128x128 weight quantizer.  One 256-thread block per (nb, kb) block: thread
// t owns column chunk t%32 (4 floats) of rows t/32, t/32+8, ..., so each
// wave-row load covers 512 contiguous bytes.  The 64 values stay in
// registers between the max pass and the encode pass.
//   w (N,K) fp32 -> wq (N,K) u8, sb [ceil(N/128)][K/128] fp32
template <bool POW2>
__global__ __launch_bounds__(256) void quant_128x128_kernel(const float* __restrict__ w,
                                                            uint8_t* __restrict__ wq,
                                                            float* __restrict__ sb, int64_t N,
                                                            int64_t K) {
    __shared__ float wave_max[4];
    const int64_t KB = K / 128;
    const int64_t nb = blockIdx.x / KB, kb = blockIdx.x - (int64_t)(blockIdx.x / KB) * KB;
    const int c = threadIdx.x & 31, r0 = threadIdx.x >> 5;
    const int64_t n0 = nb * 128;
    float4 v[16];
    float amax = 0.0f;
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t n = n0 + r0 + 8 * i;
        if (n < N) {
            v[i] = *reinterpret_cast<const float4*>(w + n * K + kb * 128 + c * 4);
            amax = fmaxf(amax, fmaxf(fmaxf(fabsf(v[i].x), fabsf(v[i].y)),
                                     fmaxf(fabsf(v[i].z), fabsf(v[i].w))));
        } else {
            v[i] = make_float4(0.f, 0.f, 0.f, 0.f);
        }
    }
#pragma unroll
    for (int off = 32; off >= 1; off >>= 1) amax = fmaxf(amax, __shfl_xor(amax, off, 64));
    if ((threadIdx.x & 63) == 0) wave_max[threadIdx.x >> 6] = amax;
    __syncthreads();
    amax = fmaxf(fmaxf(wave_max[0], wave_max[1]), fmaxf(wave_max[2], wave_max[3]));
    const float s = group_scale(amax, POW2);
#pragma unroll
    for (int i = 0; i < 16; ++i) {
        const int64_t n = n0 + r0 + 8 * i;
        if (n < N) {
            const uint32_t q = cvt_e4m3x4(v[i].x / s, v[i].y / s, v[i].z / s, v[i].w / s);
            *reinterpret_cast<uint32_t*>(wq + n * K + kb * 128 + c * 4) = q;
        }
    }
    if (threadIdx.x == 0) sb[nb * KB + kb] = s;
}

}  // namespace fp8k
