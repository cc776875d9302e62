/*
 * oracle.h -- plain, slow CPU reference for the fine-grained block-scaled
 * E4M3 GEMM (Y = X * W^T) and its quantizers.
 *
 * TEST INFRASTRUCTURE ONLY.  Only the test-suite, the smoke check and the
 * benchmark's CPU-baseline leg may load this library.  The GPU product path
 * never calls it, links it or shares code with it.
 *
 * Sources (page title, section):
 *   [DG]  "DeepGEMM 完全拆解：300 行 FP8 GEMM 内核，如何逼近 Hopper 的算力峰值"
 *   [TC]  "GPU GEMM 优化完全拆解(四): tcgen05 与 Blackwell", section 六 (6.1)
 *   [MLC] "Blackwell Tensor Core: tcgen05.mma", section "Block-Scaled MMA"
 *
 * MXFP8 (the MX variant): X and W both carry one E8M0 byte per 1x32 group
 * along K, laid out (rows, K/32) row-major; see oracle_quant_mx.
 *
 * Layouts (all row-major, element offsets):
 *   X   fp32 (M, K)            Xq  u8 (M, K)           sa fp32 [K/128][M]
 *   W   fp32 (N, K)            Wq  u8 (N, K)           sb fp32 [ceil(N/128)][K/128]
 *   Y   fp64 (M, N)
 * K must be a multiple of 128 for every block-scaled call (the scale
 * granularity along K) and of 32 for the MX calls.
 */
#ifndef FP8_ORACLE_H
#define FP8_ORACLE_H
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

#define ORACLE_FLAG_UE8M0 1u

/* E4M3 (OCP "E4M3FN": bias 7, largest finite 448, no infinities). */
double  oracle_e4m3_decode(uint8_t code);
uint8_t oracle_e4m3_encode(float v);
void    oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out);

/* Per-group scale from the group's absolute maximum. */
float   oracle_scale_from_amax(float amax, uint32_t flags);

/* 1x128 activation groups; returns 0 on success, -1 on bad shape. */
int oracle_quant_1x128(const float* x, int64_t M, int64_t K, uint32_t flags,
                       uint8_t* xq, float* sa);
/* 128x128 weight blocks (ragged at the N edge). */
int oracle_quant_128x128(const float* w, int64_t N, int64_t K, uint32_t flags,
                         uint8_t* wq, float* sb);

/* Dense NT GEMM, every element, FP64 result. */
int oracle_gemm_nt(const uint8_t* xq, const float* sa, const uint8_t* wq,
                   const float* sb, int64_t M, int64_t N, int64_t K,
                   uint32_t flags, double* y);

/* Dense NT GEMM on a list of (m, n) pairs: y[i] = Y[m[i], n[i]]. */
int oracle_gemm_nt_elems(const uint8_t* xq, const float* sa, const uint8_t* wq,
                         const float* sb, int64_t M, int64_t N, int64_t K,
                         uint32_t flags, const int64_t* m_idx,
                         const int64_t* n_idx, int64_t count, double* y);

/* Grouped, contiguous layout.  Rows whose expert index is outside [0,E), or
 * differs from the expert of their aligned 128-row block, are not written
 * (written[r] = 0); every other row is computed (written[r] = 1). */
int oracle_grouped_contiguous(const uint8_t* xq, const float* sa,
                              const uint8_t* wq, const float* sb,
                              const int32_t* m_indices, int64_t M, int64_t N,
                              int64_t K, int32_t E, uint32_t flags, double* y,
                              uint8_t* written);

/* Contract check for the contiguous layout: returns the number of aligned
 * 128-row blocks holding more than one distinct expert index in [0,E). */
int64_t oracle_contiguous_layout_violations(const int32_t* m_indices, int64_t M,
                                            int32_t E);

/* Grouped, masked layout.  X is (E*max_m, K), sa [K/128][E*max_m], W (E*N, K),
 * sb [E*N/128][K/128], y (E*max_m, N).  Row m of expert e is computed iff
 * m < clamp(masked_m[e], 0, max_m); written[] marks the computed rows. */
int oracle_grouped_masked(const uint8_t* xq, const float* sa, const uint8_t* wq,
                          const float* sb, const int32_t* masked_m, int32_t E,
                          int64_t max_m, int64_t N, int64_t K, uint32_t flags,
                          double* y, uint8_t* written);

/* MXFP8: one E8M0 scale byte per 1x32 group along K (both operands).
 * x (R, K) fp32 -> q u8 (R, K), e u8 (R, K/32); K must be a multiple of 32. */
int oracle_quant_mx(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e);
/* Y (M, N) fp64 = MX X * W^T; xq (M, K), ea (M, K/32), wq (N, K), eb (N, K/32). */
int oracle_gemm_mx(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                   const uint8_t* eb, int64_t M, int64_t N, int64_t K, double* y);
int oracle_gemm_mx_elems(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                         const uint8_t* eb, int64_t M, int64_t N, int64_t K,
                         const int64_t* m_idx, const int64_t* n_idx, int64_t count,
                         double* y);

/* MXFP4 (weights): E2M1 nibbles, one E8M0 scale byte per 1x32 group.
 * x (R, K) fp32 -> q u8 (R, K/2) (element k in byte k/2, low nibble for even
 * k), e u8 (R, K/32); K must be a multiple of 32. */
double  oracle_e2m1_decode(uint8_t code);
uint8_t oracle_e2m1_encode(float v);
int oracle_quant_mxfp4(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e);
/* Y (M, N) fp64 = X * W^T, X MXFP8 (xq (M, K), ea (M, K/32)), W MXFP4
 * (wq (N, K/2), eb (N, K/32)). */
int oracle_gemm_mx_w4(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                      const uint8_t* eb, int64_t M, int64_t N, int64_t K, double* y);
int oracle_gemm_mx_w4_elems(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                            const uint8_t* eb, int64_t M, int64_t N, int64_t K,
                            const int64_t* m_idx, const int64_t* n_idx, int64_t count,
                            double* y);

/* Number of OpenMP threads the oracle will use. */
int oracle_num_threads(void);
void oracle_set_num_threads(int n);

#ifdef __cplusplus
}
#endif
#endif
