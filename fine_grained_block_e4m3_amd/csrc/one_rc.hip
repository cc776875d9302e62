#include "kernels_exact.h"
template __global__ void fp8k::gemm_exact_kernel<256, 256, 4, 2, 0, false, 2, false>(
    const uint8_t* __restrict__, const float* __restrict__, const uint8_t* __restrict__,
    const float* __restrict__, uint16_t* __restrict__, const int32_t* __restrict__,
    const int32_t* __restrict__, fp8k::GemmParams);
