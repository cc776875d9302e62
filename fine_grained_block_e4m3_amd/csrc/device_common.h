// device_common.h -- small gfx950 device helpers shared by the kernels of
// libfp8gemm.so.  gfx950 only: no portability layer.
#pragma once

#include <hip/hip_runtime.h>
#include <stdint.h>

namespace fp8k {

typedef int   i32x2 __attribute__((ext_vector_type(2)));
typedef int   i32x4 __attribute__((ext_vector_type(4)));
typedef int   i32x8 __attribute__((ext_vector_type(8)));
typedef float f32x4 __attribute__((ext_vector_type(4)));
typedef float f32x16 __attribute__((ext_vector_type(16)));
typedef __bf16 bf16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x2 __attribute__((ext_vector_type(2)));
typedef _Float16 f16x8 __attribute__((ext_vector_type(8)));

#define FP8K_LDS __attribute__((address_space(3)))
// Lambdas of the kernels are always inlined: an out-of-line call would pass
// wave-uniform values (LDS addresses, buffer resources) in VGPRs.
#define FP8K_INLINE __attribute__((always_inline))

// Wave-uniform value (moves it to a scalar register).
__device__ __forceinline__ int uniform(int v) { return __builtin_amdgcn_readfirstlane(v); }
__device__ __forceinline__ uint64_t uniform_u64(uint64_t v) {
    const uint32_t lo = (uint32_t)uniform((int)(uint32_t)v), hi = (uint32_t)uniform((int)(uint32_t)(v >> 32));
    return ((uint64_t)hi << 32) | lo;
}

// Two FP32 values to packed E4M3 bytes with the hardware converter
// (round-to-nearest-even, OCP E4M3FN on gfx950), placed in the low (hi=false)
// or high (hi=true) half of `old`.
__device__ __forceinline__ int cvt_e4m3x2(float a, float b, int old, bool hi) {
    return hi ? __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, true)
              : __builtin_amdgcn_cvt_pk_fp8_f32(a, b, old, false);
}

// Four FP32 values to four E4M3 bytes (little-endian order a, b, c, d).
__device__ __forceinline__ uint32_t cvt_e4m3x4(float a, float b, float c, float d) {
    int v = cvt_e4m3x2(a, b, 0, false);
    v = cvt_e4m3x2(c, d, v, true);
    return (uint32_t)v;
}

// Two FP32 values to packed BF16 (hardware round-to-nearest-even).
__device__ __forceinline__ uint32_t pack_bf16x2(float a, float b) {
    bf16x2 r;
    r[0] = (__bf16)a;
    r[1] = (__bf16)b;
    return __builtin_bit_cast(uint32_t, r);
}

// Scale of one quantization group: fl32(max(amax, 1e-4) / 448), correctly
// rounded IEEE division; with `pow2` the next power of two at or above it.
__device__ __forceinline__ float group_scale(float amax, bool pow2) {
    float a = amax > 1e-4f ? amax : 1e-4f;
    float s = a / 448.0f;
    if (pow2) {
        uint32_t bits = __float_as_uint(s);
        if (bits & 0x007FFFFFu) bits = ((bits >> 23) + 1u) << 23;
        s = __uint_as_float(bits);
    }
    return s;
}

// Biased exponent byte of an FP32 scale: its E8M0 encoding when the scale is
// a power of two.
__device__ __forceinline__ int e8m0_of(float s) {
    return (int)((__float_as_uint(s) >> 23) & 0xFFu);
}

// Eight E4M3 bytes (w0 bytes 0..3, then w1 bytes 0..3) widened to FP16 with
// the hardware converter at scale 1.  Exact: every E4M3 value (4 significant
// bits, 2^-9 .. 448) is an FP16 value.
__device__ __forceinline__ f16x8 e4m3x8_to_f16(int w0, int w1) {
    const f16x2 a = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w0, 1.0f, false);
    const f16x2 b = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w0, 1.0f, true);
    const f16x2 c = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w1, 1.0f, false);
    const f16x2 d = __builtin_amdgcn_cvt_scalef32_pk_f16_fp8((unsigned)w1, 1.0f, true);
    return f16x8{a[0], a[1], b[0], b[1], c[0], c[1], d[0], d[1]};
}

}  // namespace fp8k
