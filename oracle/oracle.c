/*
 * oracle.c -- plain, slow, obviously-correct CPU reference for the
 * fine-grained block-scaled E4M3 GEMM and its quantizers.
 *
 * TEST INFRASTRUCTURE ONLY: loaded by the tests, the smoke check and the
 * benchmark's CPU-baseline leg, never by the GPU product path.  It shares no
 * code, header, table or constant generator with the GPU library.
 *
 * Precision: quantization decisions are taken in IEEE binary32 (the scales and
 * inputs are FP32 on the DeepGEMM page); every GEMM sum is taken in binary64,
 * where the 128-wide block partials are exact (see oracle_block_partial).
 *
 * Build: gcc -O2 -std=c99 -fopenmp -ffp-contract=off -fno-fast-math (SSE
 * arithmetic on x86-64, so binary32 operations round exactly once).
 */
#include "oracle.h"

#include <math.h>
#include <stdlib.h>
#include <string.h>
#ifdef _OPENMP
#include <omp.h>
#endif

#define GROUP 128 /* scale granularity along K, and the weight block edge */

/* ------------------------------------------------------------------------ */
/* E4M3 codec                                                                */
/* ------------------------------------------------------------------------ */

/*
 * Decode one E4M3 byte.  DeepGEMM page, section "FP8 的诱惑": E4M3 has 4
 * exponent bits and 3 mantissa bits with largest value 448; section
 * "离群值如何摧毁 per-tensor 量化": smallest subnormal on the order of 2^-9.
 * OCP E4M3FN: bias 7, exponent field 0 is subnormal, the all-ones pattern
 * S.1111.111 is NaN, there are no infinities.
 *   normal    (-1)^s * 2^(e-7) * (1 + m/8) = (-1)^s * (8+m) * 2^(e-10)
 *   subnormal (-1)^s * 2^(-6)  * (m/8)     = (-1)^s * m * 2^-9
 */
double oracle_e4m3_decode(uint8_t code)
{
    int s = code >> 7, e = (code >> 3) & 15, m = code & 7;
    double mag;
    if (e == 15 && m == 7) return NAN;
    if (e == 0)
        mag = ldexp((double)m, -9);
    else
        mag = ldexp((double)(8 + m), e - 10);
    return s ? -mag : mag;
}

/*
 * Encode a binary32 value: the nearest E4M3 value, ties to the code with an
 * even mantissa (bit 0 clear), magnitudes of 448 and above saturate to 448,
 * the sign is kept (so -0 and negative underflow give 0x80).  The page fixes
 * the format but not the rounding; round-to-nearest-even with saturation is
 * the plain reading.
 *
 * Brute force over the 127 non-negative finite codes.  The distance test is
 * exact in binary64: if |v| >= 2^-10 both |v| and every code are multiples of
 * 2^-33 below 2^9, so |v| - code fits in 43 bits; if |v| < 2^-10 the distance
 * to 0 is |v| itself and the rounded distance to any other code is >= 2^-10.
 */
uint8_t oracle_e4m3_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x80 : 0x00;
    double a = fabs((double)v);
    int best = 0, c;
    double best_d;
    if (isnan(v)) return (uint8_t)(sign | 0x7F);
    if (a >= 448.0) return (uint8_t)(sign | 0x7E);
    best_d = a; /* distance to code 0x00 (+0) */
    for (c = 1; c <= 0x7E; ++c) {
        double d = fabs(a - oracle_e4m3_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

void oracle_e4m3_encode_array(const float* v, int64_t n, uint8_t* out)
{
    int64_t i;
#pragma omp parallel for schedule(static)
    for (i = 0; i < n; ++i) out[i] = oracle_e4m3_encode(v[i]);
}

/* ------------------------------------------------------------------------ */
/* Quantizers                                                                */
/* ------------------------------------------------------------------------ */

/*
 * Scale of one group.  DeepGEMM page, section "离群值如何摧毁 per-tensor
 * 量化": the scale maps the group's absolute maximum onto 448 and is computed
 * online from that group alone.  Readings: s = fl32(amax / 448) with one
 * IEEE division; amax is floored at 1e-4 so an all-zero group gets a finite
 * scale.  With ORACLE_FLAG_UE8M0 (the same section: Blackwell's MXFP8 wants
 * power-of-two UE8M0 scales) s is rounded up to the next power of two by
 * dropping a nonzero mantissa and raising the exponent by one.
 */
float oracle_scale_from_amax(float amax, uint32_t flags)
{
    float a = amax > 1e-4f ? amax : 1e-4f;
    float s = a / 448.0f;
    if (flags & ORACLE_FLAG_UE8M0) {
        uint32_t bits;
        memcpy(&bits, &s, 4);
        if (bits & 0x007FFFFFu) bits = ((bits >> 23) + 1u) << 23;
        memcpy(&s, &bits, 4);
    }
    return s;
}

/*
 * Activation quantizer, one scale per 1x128 tile of a row.  DeepGEMM page,
 * section "离群值如何摧毁 per-tensor 量化": activations are grouped 1x128
 * (one token, 128 channels).  Section "为什么只做 NT 布局": the activation
 * scales (M, K/128) are handed over transposed as (K/128, M).
 *   q = E4M3(fl32(x / s)),  sa[kb][m] = s.
 */
int oracle_quant_1x128(const float* x, int64_t M, int64_t K, uint32_t flags,
                       uint8_t* xq, float* sa)
{
    int64_t m, KB;
    if (M < 0 || K < 0 || K % GROUP) return -1;
    KB = K / GROUP;
#pragma omp parallel for schedule(static)
    for (m = 0; m < M; ++m) {
        int64_t kb, k;
        for (kb = 0; kb < KB; ++kb) {
            const float* g = x + m * K + kb * GROUP;
            float amax = 0.0f, s;
            for (k = 0; k < GROUP; ++k) {
                float a = fabsf(g[k]);
                if (a > amax) amax = a;
            }
            s = oracle_scale_from_amax(amax, flags);
            sa[kb * M + m] = s;
            for (k = 0; k < GROUP; ++k)
                xq[m * K + kb * GROUP + k] = oracle_e4m3_encode(g[k] / s);
        }
    }
    return 0;
}

/*
 * Weight quantizer, one scale per 128x128 block.  DeepGEMM page, section
 * "离群值如何摧毁 per-tensor 量化": weights are grouped 128 input channels by
 * 128 output channels.  The last block row is ragged when N % 128 != 0.
 *   sb[nb][kb] = s of block (nb, kb).
 */
int oracle_quant_128x128(const float* w, int64_t N, int64_t K, uint32_t flags,
                         uint8_t* wq, float* sb)
{
    int64_t NB, KB, blk;
    if (N < 0 || K < 0 || K % GROUP) return -1;
    NB = (N + GROUP - 1) / GROUP;
    KB = K / GROUP;
#pragma omp parallel for schedule(static)
    for (blk = 0; blk < NB * KB; ++blk) {
        int64_t nb = blk / KB, kb = blk % KB;
        int64_t n0 = nb * GROUP, n1 = n0 + GROUP < N ? n0 + GROUP : N;
        int64_t n, k;
        float amax = 0.0f, s;
        for (n = n0; n < n1; ++n)
            for (k = kb * GROUP; k < (kb + 1) * GROUP; ++k) {
                float a = fabsf(w[n * K + k]);
                if (a > amax) amax = a;
            }
        s = oracle_scale_from_amax(amax, flags);
        sb[nb * KB + kb] = s;
        for (n = n0; n < n1; ++n)
            for (k = kb * GROUP; k < (kb + 1) * GROUP; ++k)
                wq[n * K + k] = oracle_e4m3_encode(w[n * K + k] / s);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* GEMM                                                                      */
/* ------------------------------------------------------------------------ */

/* With ORACLE_FLAG_UE8M0 the GEMM reads only the exponent of each scale
 * (the value 2^(e-127) of its biased exponent field e); without it, the full
 * FP32 value. */
static double eff_scale(float s, uint32_t flags)
{
    if (flags & ORACLE_FLAG_UE8M0) {
        uint32_t bits;
        memcpy(&bits, &s, 4);
        return ldexp(1.0, (int)((bits >> 23) & 0xFFu) - 127);
    }
    return (double)s;
}

/*
 * Sum over one 128-wide K block of decoded products, in binary64.  Exact:
 * every E4M3 value is j * 2^-9 with |j| <= 229376 < 2^18, so each product is
 * an integer multiple of 2^-18 below 2^36 * 2^-18 and the 128-term sum is a
 * multiple of 2^-18 below 2^43 * 2^-18, which binary64 holds exactly.
 * DeepGEMM page, section "细粒度缩放在 GEMM 层面引爆的两个问题": the product of
 * two E4M3 values is exact, all error comes from accumulation.
 */
static double oracle_block_partial(const uint8_t* a, const uint8_t* b,
                                   const double* dec)
{
    double p = 0.0;
    int k;
    for (k = 0; k < GROUP; ++k) p += dec[a[k]] * dec[b[k]];
    return p;
}

/*
 * One output element of the block-scaled GEMM.  GEMM definition with block
 * scale factors: tcgen05 page, section 6.1, D_ij = C_ij + sum_k (A_ik *
 * SFA_i,floor(k/SV)) (B_jk * SFB_j,floor(k/SV)); scale indexing per output
 * (m, n) uses SFA[m, sfk] and SFB[n, sfk] (mlc.ai page, "Block-Scaled MMA").
 * Here SV = 128, SFA = sa[kb][m] and SFB for row n of W is its 128x128 block's
 * sb[n/128][kb].  DeepGEMM page, section "主循环骨架": each 128-K block's
 * partial is multiplied by sA * sB and added to a full-precision accumulator.
 */
static double oracle_dot(const uint8_t* xq_row, const float* sa, int64_t M,
                         int64_t m, const uint8_t* wq_row, const float* sb,
                         int64_t n, int64_t K, uint32_t flags,
                         const double* dec)
{
    int64_t KB = K / GROUP, kb;
    double acc = 0.0;
    for (kb = 0; kb < KB; ++kb) {
        double p = oracle_block_partial(xq_row + kb * GROUP,
                                        wq_row + kb * GROUP, dec);
        double s = eff_scale(sa[kb * M + m], flags) *
                   eff_scale(sb[(n / GROUP) * KB + kb], flags); /* exact */
        acc += s * p;
    }
    return acc;
}

static void fill_decode_table(double* dec)
{
    int c;
    for (c = 0; c < 256; ++c) dec[c] = oracle_e4m3_decode((uint8_t)c);
}

/* Dense NT GEMM, Y = X * W^T.  DeepGEMM page, section "为什么只做 NT 布局":
 * X is (M, K) row-major, W is stored as (N, K) with K contiguous. */
int oracle_gemm_nt(const uint8_t* xq, const float* sa, const uint8_t* wq,
                   const float* sb, int64_t M, int64_t N, int64_t K,
                   uint32_t flags, double* y)
{
    double dec[256];
    int64_t m;
    if (M < 0 || N < 0 || K < 0 || K % GROUP) return -1;
    fill_decode_table(dec);
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n)
            y[m * N + n] = oracle_dot(xq + m * K, sa, M, m, wq + n * K, sb, n,
                                      K, flags, dec);
    }
    return 0;
}

int oracle_gemm_nt_elems(const uint8_t* xq, const float* sa, const uint8_t* wq,
                         const float* sb, int64_t M, int64_t N, int64_t K,
                         uint32_t flags, const int64_t* m_idx,
                         const int64_t* n_idx, int64_t count, double* y)
{
    double dec[256];
    int64_t i;
    if (M < 0 || N < 0 || K < 0 || K % GROUP || count < 0) return -1;
    for (i = 0; i < count; ++i)
        if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N)
            return -1;
    fill_decode_table(dec);
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i) {
        int64_t m = m_idx[i], n = n_idx[i];
        y[i] = oracle_dot(xq + m * K, sa, M, m, wq + n * K, sb, n, K, flags,
                          dec);
    }
    return 0;
}

/* ------------------------------------------------------------------------ */
/* Grouped GEMMs (MoE experts)                                               */
/* ------------------------------------------------------------------------ */

/* Expert of the aligned 128-row block holding row r: the first index in that
 * block that names an expert in [0, E), or -1 if none does. */
static int32_t block_expert(const int32_t* idx, int64_t M, int64_t r, int32_t E)
{
    int64_t b0 = (r / GROUP) * GROUP, b1 = b0 + GROUP < M ? b0 + GROUP : M, i;
    for (i = b0; i < b1; ++i)
        if (idx[i] >= 0 && idx[i] < E) return idx[i];
    return -1;
}

/*
 * Contiguous layout.  DeepGEMM page, section "分组 GEMM 的两种布局": the
 * tokens of each expert are concatenated along M into one segment, N and K
 * are shared by all experts, and each segment is aligned to the GEMM's M
 * block (the alignment query).  Reading: a per-row int32 expert index, -1 on
 * padding rows; padding rows are not written.  Expert e's weights are rows
 * [e*N, (e+1)*N) of wq and its scales rows [e*N/128, (e+1)*N/128) of sb.
 */
int oracle_grouped_contiguous(const uint8_t* xq, const float* sa,
                              const uint8_t* wq, const float* sb,
                              const int32_t* m_indices, int64_t M, int64_t N,
                              int64_t K, int32_t E, uint32_t flags, double* y,
                              uint8_t* written)
{
    double dec[256];
    int64_t r, KB;
    if (M < 0 || N < 0 || K < 0 || E < 0 || K % GROUP || N % GROUP) return -1;
    KB = K / GROUP;
    fill_decode_table(dec);
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < M; ++r) {
        int32_t e = m_indices[r];
        int64_t n;
        written[r] = 0;
        if (e < 0 || e >= E) continue;
        if (block_expert(m_indices, M, r, E) != e) continue;
        written[r] = 1;
        for (n = 0; n < N; ++n)
            y[r * N + n] = oracle_dot(xq + r * K, sa, M, r,
                                      wq + ((int64_t)e * N + n) * K,
                                      sb + (int64_t)e * (N / GROUP) * KB, n, K,
                                      flags, dec);
    }
    return 0;
}

int64_t oracle_contiguous_layout_violations(const int32_t* m_indices, int64_t M,
                                            int32_t E)
{
    int64_t b, bad = 0;
    for (b = 0; b < M; b += GROUP) {
        int64_t i, end = b + GROUP < M ? b + GROUP : M;
        int32_t first = -1;
        for (i = b; i < end; ++i) {
            int32_t e = m_indices[i];
            if (e < 0 || e >= E) continue;
            if (first < 0) first = e;
            else if (e != first) { ++bad; break; }
        }
    }
    return bad;
}

/*
 * Masked layout.  DeepGEMM page, section "分组 GEMM 的两种布局": in decode the
 * host does not know how many tokens each expert receives, so a mask marks the
 * valid positions and only those are computed; section "统一块调度器与
 * rasterization": the scheduler covers only each expert's valid rows.
 * Reading: a per-expert int32 count, clamped to [0, max_m]; rows at or past it
 * are not written.
 */
int oracle_grouped_masked(const uint8_t* xq, const float* sa, const uint8_t* wq,
                          const float* sb, const int32_t* masked_m, int32_t E,
                          int64_t max_m, int64_t N, int64_t K, uint32_t flags,
                          double* y, uint8_t* written)
{
    double dec[256];
    int64_t r, KB, MT;
    if (E < 0 || max_m < 0 || N < 0 || K < 0 || K % GROUP || N % GROUP)
        return -1;
    KB = K / GROUP;
    MT = (int64_t)E * max_m;
    fill_decode_table(dec);
#pragma omp parallel for schedule(dynamic, 1)
    for (r = 0; r < MT; ++r) {
        int64_t e = r / max_m, m = r % max_m, n;
        int64_t valid = masked_m[e];
        if (valid < 0) valid = 0;
        if (valid > max_m) valid = max_m;
        written[r] = 0;
        if (m >= valid) continue;
        written[r] = 1;
        for (n = 0; n < N; ++n)
            y[r * N + n] = oracle_dot(xq + r * K, sa, MT, r,
                                      wq + (e * N + n) * K,
                                      sb + e * (N / GROUP) * KB, n, K, flags,
                                      dec);
    }
    return 0;
}

int oracle_num_threads(void)
{
#ifdef _OPENMP
    return omp_get_max_threads();
#else
    return 1;
#endif
}

/* Threads for the following calls (n >= 1); no effect on any result: every
 * parallel loop writes disjoint outputs, each computed in a fixed order. */
void oracle_set_num_threads(int n)
{
#ifdef _OPENMP
    if (n >= 1)
        omp_set_num_threads(n);
#else
    (void)n;
#endif
}

/* ------------------------------------------------------------------------ */
/* MXFP8: E4M3 elements, one E8M0 scale per 1x32 group along K               */
/* ------------------------------------------------------------------------ */

#define MX_GROUP 32 /* elements per MX scale, along K */

/*
 * MX quantizer of a row-major (R, K) matrix, activations and weights alike.
 * tcgen05 page, sections 6.1 and 6.3: in the MX formats every 32 consecutive
 * elements along K share one scale, an E8M0 byte (a pure power of two); the
 * aside in section 5.4 names MXFP8 among the inputs of DeepGEMM's Blackwell
 * path.  The pages give no rule for choosing the scale.  Reading: the UE8M0
 * rule of the 1x128 quantizer, applied to each 32-group: s is the power of
 * two at or above fl32(max(amax, 1e-4) / 448), so no code saturates.
 *   q = E4M3(fl32(x / s)),  e[r][g] = biased exponent of s  (s = 2^(e-127)).
 */
int oracle_quant_mx(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e)
{
    int64_t r, G;
    if (R < 0 || K < 0 || K % MX_GROUP) return -1;
    G = K / MX_GROUP;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; ++r) {
        int64_t g, k;
        for (g = 0; g < G; ++g) {
            const float* v = x + r * K + g * MX_GROUP;
            float amax = 0.0f, s;
            uint32_t bits;
            for (k = 0; k < MX_GROUP; ++k) {
                float a = fabsf(v[k]);
                if (a > amax) amax = a;
            }
            s = oracle_scale_from_amax(amax, ORACLE_FLAG_UE8M0);
            memcpy(&bits, &s, 4);
            e[r * G + g] = (uint8_t)((bits >> 23) & 0xFFu);
            for (k = 0; k < MX_GROUP; ++k)
                q[r * K + g * MX_GROUP + k] = oracle_e4m3_encode(v[k] / s);
        }
    }
    return 0;
}

/*
 * One output element of the MX GEMM.  tcgen05 page, section 6.1, with
 * SV = 32, SFA[m][g] = 2^(ea[m][g]-127) and SFB[n][g] = 2^(eb[n][g]-127):
 *   Y[m][n] = sum_g SFA[m][g] * SFB[n][g] * sum_{k in group g} dec(xq[m][k]) * dec(wq[n][k]).
 * Each 32-term partial is exact in binary64 (a sub-sum of the exact 128-term
 * partials), and so is the power-of-two scale product.
 */
static double oracle_dot_mx(const uint8_t* xr, const uint8_t* ear, const uint8_t* wr,
                            const uint8_t* ebr, int64_t K, const double* dec)
{
    int64_t G = K / MX_GROUP, g;
    double acc = 0.0;
    for (g = 0; g < G; ++g) {
        double p = 0.0;
        int k;
        for (k = 0; k < MX_GROUP; ++k) p += dec[xr[g * MX_GROUP + k]] * dec[wr[g * MX_GROUP + k]];
        acc += ldexp(1.0, (int)ear[g] - 127) * ldexp(1.0, (int)ebr[g] - 127) * p;
    }
    return acc;
}

/* Dense NT MX GEMM, Y = X * W^T with xq (M, K), ea (M, K/32), wq (N, K),
 * eb (N, K/32), all row-major. */
int oracle_gemm_mx(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                   const uint8_t* eb, int64_t M, int64_t N, int64_t K, double* y)
{
    double dec[256];
    int64_t m, G;
    if (M < 0 || N < 0 || K < 0 || K % MX_GROUP) return -1;
    G = K / MX_GROUP;
    fill_decode_table(dec);
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n)
            y[m * N + n] = oracle_dot_mx(xq + m * K, ea + m * G, wq + n * K, eb + n * G, K, dec);
    }
    return 0;
}

/* The MX GEMM on a list of (m, n) pairs: y[i] = Y[m_idx[i]][n_idx[i]]. */
int oracle_gemm_mx_elems(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                         const uint8_t* eb, int64_t M, int64_t N, int64_t K,
                         const int64_t* m_idx, const int64_t* n_idx, int64_t count, double* y)
{
    double dec[256];
    int64_t i, G;
    if (M < 0 || N < 0 || K < 0 || K % MX_GROUP || count < 0) return -1;
    for (i = 0; i < count; ++i)
        if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N) return -1;
    G = K / MX_GROUP;
    fill_decode_table(dec);
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i)
        y[i] = oracle_dot_mx(xq + m_idx[i] * K, ea + m_idx[i] * G, wq + n_idx[i] * K,
                             eb + n_idx[i] * G, K, dec);
    return 0;
}

/* ------------------------------------------------------------------------ */
/* MXFP4 weights: E2M1 elements, one E8M0 scale per 1x32 group along K       */
/* ------------------------------------------------------------------------ */

/*
 * Decode one E2M1 nibble.  tcgen05 page, section 6.3: MXFP4 elements are
 * E2M1 (1 sign, 2 exponent, 1 mantissa bit) with an E8M0 scale per 32.
 * Exponent bias 1, exponent field 0 is subnormal, no infinities or NaN:
 *   normal    (-1)^s * 2^(e-1) * (1 + m/2)
 *   subnormal (-1)^s * m/2
 * giving the magnitudes 0, 0.5, 1, 1.5, 2, 3, 4, 6.
 */
double oracle_e2m1_decode(uint8_t code)
{
    int s = (code >> 3) & 1, e = (code >> 1) & 3, m = code & 1;
    double mag = e == 0 ? 0.5 * m : ldexp(1.0 + 0.5 * m, e - 1);
    return s ? -mag : mag;
}

/*
 * Encode a binary32 value to E2M1: the nearest value, ties to the code with
 * an even mantissa bit, magnitudes above 6 saturating to 6, the sign kept.
 * Brute force over the 8 magnitudes (all distances exact in binary64).
 */
uint8_t oracle_e2m1_encode(float v)
{
    uint8_t sign = signbit(v) ? 0x8 : 0x0;
    double a = fabs((double)v), best_d;
    int best = 0, c;
    if (a >= 6.0) return (uint8_t)(sign | 0x7);
    best_d = a;
    for (c = 1; c <= 7; ++c) {
        double d = fabs(a - oracle_e2m1_decode((uint8_t)c));
        if (d < best_d || (d == best_d && (c & 1) == 0)) {
            best = c;
            best_d = d;
        }
    }
    return (uint8_t)(sign | best);
}

/*
 * MXFP4 quantizer of a row-major (R, K) matrix.  Reading (as for MXFP8): the
 * scale of a 1x32 group is the power of two at or above
 * fl32(max(amax, 1e-4) / 6), 6 being the largest E2M1 magnitude, so no
 * element saturates.  Output: element k of row r in byte r*K/2 + k/2, the
 * low nibble for even k; e[r][g] = biased exponent of the group's scale.
 */
int oracle_quant_mxfp4(const float* x, int64_t R, int64_t K, uint8_t* q, uint8_t* e)
{
    int64_t r, G;
    if (R < 0 || K < 0 || K % MX_GROUP) return -1;
    G = K / MX_GROUP;
#pragma omp parallel for schedule(static)
    for (r = 0; r < R; ++r) {
        int64_t g, k;
        for (g = 0; g < G; ++g) {
            const float* v = x + r * K + g * MX_GROUP;
            float amax = 0.0f, a, s;
            uint32_t bits;
            for (k = 0; k < MX_GROUP; ++k) {
                float t = fabsf(v[k]);
                if (t > amax) amax = t;
            }
            a = amax > 1e-4f ? amax : 1e-4f;
            s = a / 6.0f;
            memcpy(&bits, &s, 4);
            if (bits & 0x007FFFFFu) bits = ((bits >> 23) + 1u) << 23;
            memcpy(&s, &bits, 4);
            e[r * G + g] = (uint8_t)((bits >> 23) & 0xFFu);
            for (k = 0; k < MX_GROUP; k += 2) {
                uint8_t lo = oracle_e2m1_encode(v[k] / s), hi = oracle_e2m1_encode(v[k + 1] / s);
                q[(r * K + g * MX_GROUP + k) / 2] = (uint8_t)(lo | (hi << 4));
            }
        }
    }
    return 0;
}

/* One element of the MXFP8 x MXFP4 GEMM: as oracle_dot_mx, with W's elements
 * E2M1 nibbles (tcgen05 page, section 6.1 with SV = 32). */
static double oracle_dot_mx_w4(const uint8_t* xr, const uint8_t* ear, const uint8_t* wr,
                               const uint8_t* ebr, int64_t K, const double* dec8,
                               const double* dec4)
{
    int64_t G = K / MX_GROUP, g;
    double acc = 0.0;
    for (g = 0; g < G; ++g) {
        double p = 0.0;
        int k;
        for (k = 0; k < MX_GROUP; ++k) {
            int64_t kk = g * MX_GROUP + k;
            uint8_t nib = (uint8_t)((wr[kk / 2] >> (4 * (kk & 1))) & 0xF);
            p += dec8[xr[kk]] * dec4[nib];
        }
        acc += ldexp(1.0, (int)ear[g] - 127) * ldexp(1.0, (int)ebr[g] - 127) * p;
    }
    return acc;
}

/* Y (M, N) = X * W^T with X MXFP8 (xq (M, K), ea (M, K/32)) and W MXFP4
 * (wq (N, K/2) packed nibbles, eb (N, K/32)); on a list of (m, n) pairs. */
int oracle_gemm_mx_w4_elems(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                            const uint8_t* eb, int64_t M, int64_t N, int64_t K,
                            const int64_t* m_idx, const int64_t* n_idx, int64_t count, double* y)
{
    double dec8[256], dec4[16];
    int64_t i, G;
    int c;
    if (M < 0 || N < 0 || K < 0 || K % MX_GROUP || count < 0) return -1;
    for (i = 0; i < count; ++i)
        if (m_idx[i] < 0 || m_idx[i] >= M || n_idx[i] < 0 || n_idx[i] >= N) return -1;
    G = K / MX_GROUP;
    fill_decode_table(dec8);
    for (c = 0; c < 16; ++c) dec4[c] = oracle_e2m1_decode((uint8_t)c);
#pragma omp parallel for schedule(static)
    for (i = 0; i < count; ++i)
        y[i] = oracle_dot_mx_w4(xq + m_idx[i] * K, ea + m_idx[i] * G, wq + n_idx[i] * (K / 2),
                                eb + n_idx[i] * G, K, dec8, dec4);
    return 0;
}

int oracle_gemm_mx_w4(const uint8_t* xq, const uint8_t* ea, const uint8_t* wq,
                      const uint8_t* eb, int64_t M, int64_t N, int64_t K, double* y)
{
    double dec8[256], dec4[16];
    int64_t m, G;
    int c;
    if (M < 0 || N < 0 || K < 0 || K % MX_GROUP) return -1;
    G = K / MX_GROUP;
    fill_decode_table(dec8);
    for (c = 0; c < 16; ++c) dec4[c] = oracle_e2m1_decode((uint8_t)c);
#pragma omp parallel for schedule(dynamic, 1)
    for (m = 0; m < M; ++m) {
        int64_t n;
        for (n = 0; n < N; ++n)
            y[m * N + n] = oracle_dot_mx_w4(xq + m * K, ea + m * G, wq + n * (K / 2), eb + n * G,
                                            K, dec8, dec4);
    }
    return 0;
}
