/*
 * fp8gemm.h -- C ABI of libfp8gemm.so: fine-grained block-scaled E4M3 GEMM
 * (Y = X * W^T, BF16 out) and its quantizers, hand-written for AMD gfx950
 * (MI355X, CDNA4).
 *
 * Sources (page title, section):
 *   [DG]  "DeepGEMM 完全拆解：300 行 FP8 GEMM 内核，如何逼近 Hopper 的算力峰值"
 *   [TC]  "GPU GEMM 优化完全拆解(四): tcgen05 与 Blackwell", section 六 (6.1)
 *   [MLC] "Blackwell Tensor Core: tcgen05.mma", section "Block-Scaled MMA"
 *
 * Common conventions
 *   - Every pointer argument is a DEVICE pointer owned by the caller.  The
 *     library never allocates, frees, retains or synchronizes; each call only
 *     enqueues kernels on `stream` (a hipStream_t, NULL = the null stream) and
 *     returns.  Outputs must not alias inputs.
 *   - E4M3 is OCP E4M3FN (bias 7, largest finite 448, NaN = S.1111.111).
 *     BF16 outputs are stored as raw uint16_t bit patterns, rounded to
 *     nearest-even.
 *   - Layouts are row-major.  The activation scale table is "MN-major":
 *     sa[kb][m] at sa + kb*M + m, kb = k/128  ([DG] "为什么只做 NT 布局": the
 *     (M, K/128) activation scales are handed over transposed as (K/128, M)).
 *     The weight scale table is sb[nb][kb] at sb + nb*(K/128) + kb, nb = n/128.
 *   - K must be a multiple of 128 (the scale granularity along K; [DG]
 *     "线程组织": the K block is fixed at 128 because scaling is per 128
 *     channels).
 *   - Errors are detected on the host before anything is enqueued:
 *       FP8_ERR_INVALID_ARG  null pointer, negative or oversized dimension,
 *                            unknown flag bit
 *       FP8_ERR_SHAPE        K % 128 != 0; N % 128 != 0 for grouped calls
 *       FP8_ERR_ALIGNMENT    a pointer not 16-byte aligned
 *       FP8_ERR_NO_DEVICE    no HIP device is usable
 *       FP8_ERR_LAUNCH       the kernel launch reported an error
 *       FP8_ERR_SCRATCH      (fp8_gemm_nt_noalloc) the problem needs more
 *                            split-K scratch than its fixed array holds
 *     A call with an empty problem (M == 0, E == 0, N == 0 ...) returns FP8_OK
 *     and enqueues nothing.  Device-side data (expert indices, valid counts)
 *     is never reported as an error: its handling is defined per call.
 *   - NaN or infinite inputs give unspecified (but in-bounds) results.
 *   - Thread safety: all calls are reentrant; the only global state is a
 *     per-device cache of the compute-unit count, filled once.
 */
#ifndef FP8GEMM_H
#define FP8GEMM_H
#include <stddef.h>
#include <stdint.h>

#ifdef __cplusplus
extern "C" {
#endif

typedef enum {
    FP8_OK = 0,
    FP8_ERR_INVALID_ARG = 1,
    FP8_ERR_SHAPE = 2,
    FP8_ERR_ALIGNMENT = 3,
    FP8_ERR_UNSUPPORTED = 4,
    FP8_ERR_NO_DEVICE = 5,
    FP8_ERR_LAUNCH = 6,
    FP8_ERR_SCRATCH = 7
} fp8_status;

/* Quantizers: round each group's scale up to a power of two (UE8M0, [DG]
 * "离群值如何摧毁 per-tensor 量化": Blackwell MXFP8 takes power-of-two UE8M0
 * scales).  GEMMs: the scales are powers of two; only the biased exponent of
 * each FP32 scale is used (value 2^(e-127)) and the block scaling runs inside
 * the matrix instruction. */
#define FP8_FLAG_UE8M0 1u

/* GEMMs only: form each 128-K block partial with the FP8 matrix instruction
 * (twice the FP16 matrix rate) instead of exactly.
 *
 * Default (flag clear): the E4M3 operands are widened to FP16, which is exact,
 * and multiplied by FP16 matrix instructions: every product is exact and
 * every sum FP32-accurate, so Y is the exact block-scaled sum up to FP32
 * accumulation and BF16 rounding, i.e. within |y - ref| <= 8e-3*|ref| +
 * 1e-3*rms(ref) of the exact value ref barring cancellation below FP32
 * precision ([DG] "细粒度缩放在 GEMM 层面引爆的两个问题": the promotion exists
 * so that the sum is accumulated at full precision).
 *
 * FP8_FLAG_FAST_ACCUM: the FP8 instruction of gfx950 truncates, within each
 * group of 8 consecutive K, every product toward zero to a multiple of
 * 2^(E-13), 2^E being the group's largest product magnitude (measured; the
 * analog of the limited FP8 accumulation precision the DeepGEMM page reports
 * for H800 tensor cores).  Per output element the error therefore stays below
 *   2^-10 * sum over 8-groups g of sa*sb * max_{k in g} |x[m][k]| * max_{k in g} |w[n][k]|
 * (decoded E4M3 values, the scales of g's block) plus FP32/BF16 rounding,
 * which can exceed the tolerance above where the sum cancels.  With
 * FP8_FLAG_UE8M0 the block scaling then runs inside the scaled FP8
 * instruction and the K sum stays in its FP32 accumulator. */
#define FP8_FLAG_FAST_ACCUM 2u

/*
 * Activation quantizer, 1x128 groups ([DG] "离群值如何摧毁 per-tensor 量化":
 * activations are grouped per token and per 128 channels; the scale is the
 * group's absolute maximum over 448, computed online).
 *   x   fp32 (M, K)           input
 *   xq  u8   (M, K)           output codes, q = E4M3(fl32(x / s))
 *   sa  fp32 [K/128][M]       output scales, s = fl32(max(amax, 1e-4) / 448)
 *                             (rounded up to 2^k with FP8_FLAG_UE8M0)
 */
fp8_status fp8_quant_1x128(const float* x, int64_t M, int64_t K, uint8_t* xq,
                           float* sa, uint32_t flags, void* stream);

/*
 * Weight quantizer, 128x128 blocks ([DG] same section: weights are grouped 128
 * input by 128 output channels).  The last block row is ragged when
 * N % 128 != 0.
 *   w   fp32 (N, K)                 input
 *   wq  u8   (N, K)                 output codes
 *   sb  fp32 [ceil(N/128)][K/128]   output block scales (as for sa)
 */
fp8_status fp8_quant_128x128(const float* w, int64_t N, int64_t K, uint8_t* wq,
                             float* sb, uint32_t flags, void* stream);

/*
 * Dense NT GEMM ([DG] "为什么只做 NT 布局": Y = X W^T with X (M,K) row-major and
 * W stored (N,K) K-contiguous; [TC] 6.1 block-scaled GEMM definition;
 * [DG] "主循环骨架": FP32 partial sums of each 128-K block are multiplied by
 * sA*sB and added to a full-precision accumulator).
 *   Y[m][n] = sum_kb sa[kb][m] * sb[n/128][kb] * sum_{k in kb} xq[m][k]*wq[n][k]
 *   xq u8 (M,K), sa fp32 [K/128][M], wq u8 (N,K), sb fp32 [ceil(N/128)][K/128],
 *   y  bf16 bits (M,N).
 * flags: FP8_FLAG_UE8M0, FP8_FLAG_FAST_ACCUM.  Uses the caller's buffers only
 * (equivalent to fp8_gemm_nt_ws with no workspace).
 * Scales are finite and non-negative; a zero scale is taken to come with
 * all-zero codes in its group (the quantizers never write one: their scales
 * are at least 1e-4/448).  The default path keeps its accumulator in units
 * of the current block's scale product and skips a zero factor, so nonzero
 * codes under a zero scale are outside its contract.
 */
fp8_status fp8_gemm_nt(const uint8_t* xq, const float* sa, const uint8_t* wq,
                       const float* sb, uint16_t* y, int64_t M, int64_t N,
                       int64_t K, uint32_t flags, void* stream);

/*
 * fp8_gemm_nt with a caller-owned device workspace.  For decode-sized M (the
 * default path: M <= 64; FP8_FLAG_FAST_ACCUM: M <= 32) and fewer 96-column
 * tiles than compute units, the decode kernel splits K over up to 8
 * workgroups per tile when `workspace` holds their FP32 partial sums, and a
 * second kernel adds them in split order (the same result for the same
 * split).  fp8_gemm_workspace_size() gives the bytes that enable
 * the split for a shape on the current device (0: no split).  With a smaller
 * or no workspace the GEMM runs unsplit.  The workspace is only read and
 * written by this call's kernels, in stream order; calls that overlap on one
 * workspace race.  workspace_bytes > 0 needs a non-NULL, 16-byte aligned
 * workspace.
 */
fp8_status fp8_gemm_nt_ws(const uint8_t* xq, const float* sa, const uint8_t* wq,
                          const float* sb, uint16_t* y, int64_t M, int64_t N,
                          int64_t K, uint32_t flags, void* workspace,
                          size_t workspace_bytes, void* stream);

/*
 * fp8_gemm_nt for callers that cannot allocate (code under graph capture,
 * tight serving loops, harnesses that forbid hipMalloc): fp8_gemm_nt_ws with
 * the split-K workspace taken from a fixed 8 MiB device array inside the
 * library (one per GPU, loaded with the library, held until the process
 * ends) instead of the caller's memory.  Calls no hipMalloc, hipFree or
 * other allocating routine; the first call on a device looks up that
 * device's array.  The result equals fp8_gemm_nt_ws with a workspace of
 * fp8_gemm_workspace_size() bytes.  A shape whose split needs more than the
 * array (none on a device of up to 341 compute units) returns
 * FP8_ERR_SCRATCH before any launch.  Every call on one GPU shares the
 * array: calls that overlap on one GPU (several streams, or several host
 * threads) race on it and must be ordered by the caller.  Each split writes
 * every partial sum it covers before the reduction reads it, so nothing
 * needs clearing between calls.
 */
fp8_status fp8_gemm_nt_noalloc(const uint8_t* xq, const float* sa, const uint8_t* wq,
                               const float* sb, uint16_t* y, int64_t M, int64_t N,
                               int64_t K, uint32_t flags, void* stream);

/* Workspace bytes with which fp8_gemm_nt_ws splits K for this shape and these
 * flags on the current device (0 when it does not split, or on bad
 * arguments). */
size_t fp8_gemm_workspace_size(int64_t M, int64_t N, int64_t K, uint32_t flags);

/*
 * Dense NT GEMM whose output is quantized for the next GEMM in the epilogue
 * ([DG] "为什么只做 NT 布局": DeepGEMM leaves the activation quantization to
 * the caller, to be fused into the kernel that produces the activations).
 * Y is computed as by fp8_gemm_nt and, instead of BF16, written as the 1x128
 * activation quantizer would write it, from the FP32 accumulator:
 *   yq  u8   (M,N)         E4M3 codes, E4M3(acc / s)
 *   sy  fp32 [N/128][M]    s = fl32(max(amax, 1e-4)/448) over the 128
 *                          columns of the group (rounded up to 2^k with
 *                          FP8_FLAG_UE8M0, which also marks the input scales)
 * so (yq, sy) is the (xq, sa) of a following fp8_gemm_nt with K = N.
 * N % 128 == 0; flags as for fp8_gemm_nt.
 */
fp8_status fp8_gemm_nt_qout(const uint8_t* xq, const float* sa, const uint8_t* wq,
                            const float* sb, uint8_t* yq, float* sy, int64_t M,
                            int64_t N, int64_t K, uint32_t flags, void* stream);

/*
 * Grouped GEMM, contiguous layout ([DG] "分组 GEMM 的两种布局": the tokens of
 * each expert form one segment along M, N and K are shared by all experts,
 * each segment is aligned to the M block reported by
 * fp8_get_mk_alignment_for_contiguous_layout()).
 *   xq u8 (M,K), sa fp32 [K/128][M], m_indices int32 (M) on the device,
 *   wq u8 (E,N,K), sb fp32 (E, N/128, K/128), y bf16 bits (M,N).  N % 128 == 0.
 *   Row r uses expert m_indices[r].  Each aligned 128-row block is computed
 *   with the expert of its first row whose index lies in [0,E); a row is
 *   written only if its index equals that expert, every other row (padding
 *   rows with -1, out-of-range indices, rows of another expert in the same
 *   block) is left untouched.
 */
fp8_status fp8_grouped_gemm_contiguous(const uint8_t* xq, const float* sa,
                                       const uint8_t* wq, const float* sb,
                                       const int32_t* m_indices, uint16_t* y,
                                       int64_t M, int64_t N, int64_t K,
                                       int32_t E, uint32_t flags, void* stream);

/*
 * Grouped GEMM, masked layout ([DG] "分组 GEMM 的两种布局": decode with counts
 * unknown to the host, only the valid positions are computed; [DG]
 * "统一块调度器与 rasterization": the scheduler skips experts without work and
 * covers only valid rows).
 *   xq u8 (E,max_m,K), sa fp32 [K/128][E*max_m], masked_m int32 (E) on the
 *   device, wq u8 (E,N,K), sb fp32 (E,N/128,K/128), y bf16 bits (E,max_m,N).
 *   N % 128 == 0.  Row m of expert e is written iff m < clamp(masked_m[e], 0,
 *   max_m); every other row of y is left untouched and rows of xq past the
 *   count need not hold finite values.
 */
fp8_status fp8_grouped_gemm_masked(const uint8_t* xq, const float* sa,
                                   const uint8_t* wq, const float* sb,
                                   const int32_t* masked_m, uint16_t* y,
                                   int32_t E, int64_t max_m, int64_t N,
                                   int64_t K, uint32_t flags, void* stream);

/*
 * MXFP8 quantizer, for activations and weights alike ([TC] sections 6.1 and
 * 6.3: the MX formats share one E8M0 scale, a pure power of two, over 32
 * consecutive elements along K; [TC] 5.4 names MXFP8 among the inputs of
 * DeepGEMM's Blackwell path).  The scale of a group is the power of two at or
 * above max(amax, 1e-4) / 448 (the pages give no rule; this is the UE8M0 rule
 * of the 1x128 groups), so no code saturates.  The scale bytes are packed and
 * transposed ([TC] 5.4: DeepGEMM's Blackwell path takes packed UE8M0 scales
 * in a transposed layout): the 4 bytes of the groups of one 128-K block of a
 * row form one dword, and the dwords are laid out [K/128][R].
 *   x  fp32 (R, K)          input, K % 128 == 0
 *   q  u8   (R, K)          output codes, q = E4M3(x / s)
 *   e  u32  [K/128][R]      output scales: byte t of e[kb*R + r] is the scale
 *                           byte b of group 4*kb + t of row r, s = 2^(b - 127)
 */
fp8_status fp8_quant_mx(const float* x, int64_t R, int64_t K, uint8_t* q,
                        uint32_t* e, void* stream);

/*
 * Dense NT GEMM on MXFP8 operands ([TC] 6.1 with scale vector length 32:
 *   Y[m][n] = sum_g 2^(ea(m,g)-127) * 2^(eb(n,g)-127)
 *                   * sum_{k in group g} xq[m][k] * wq[n][k]).
 *   xq u8 (M,K), ea u32 [K/128][M], wq u8 (N,K), eb u32 [K/128][N] (packed as
 *   fp8_quant_mx writes them; ea[kb][m] byte t is the exponent byte of group
 *   4*kb + t), y bf16 bits (M,N); K % 128 == 0.  Every lane of the scaled
 *   matrix instruction holds one 32-group of its row and takes that group's
 *   byte as its scale, so the whole K sum stays in the instruction's FP32
 *   accumulator.  Accuracy: that of the FP8 instruction (the bound stated at
 *   FP8_FLAG_FAST_ACCUM, with each 32-group's scales).  flags must be 0.
 */
fp8_status fp8_gemm_nt_mx(const uint8_t* xq, const uint32_t* ea,
                          const uint8_t* wq, const uint32_t* eb, uint16_t* y,
                          int64_t M, int64_t N, int64_t K, uint32_t flags,
                          void* stream);

/*
 * MXFP4 weight quantizer ([TC] 6.3: MXFP4 = E2M1 elements with one E8M0 scale
 * per 32; [TC] notes on operand majors: two 4-bit values are packed per byte
 * along K).  The scale of a group is the power of two at or above
 * max(amax, 1e-4) / 6, 6 being the largest E2M1 magnitude (a reading, as for
 * MXFP8), so no element saturates; elements round to nearest, ties to even.
 *   x  fp32 (R, K)          input, K % 128 == 0
 *   q  u8   (R, K/2)        output: element k of a row in byte k/2, the even
 *                           one in the low nibble (E2M1: sign bit 3,
 *                           exponent bits 2..1, mantissa bit 0)
 *   e  u32  [K/128][R]      output scales, packed as by fp8_quant_mx
 */
fp8_status fp8_quant_mxfp4(const float* x, int64_t R, int64_t K, uint8_t* q,
                           uint32_t* e, void* stream);

/*
 * Dense NT GEMM with MXFP8 activations and MXFP4 weights (weight-only 4-bit
 * decode: half the weight bytes of MXFP8):
 *   Y[m][n] = sum_g 2^(ea(m,g)-127) * 2^(eb(n,g)-127)
 *                   * sum_{k in group g} xq[m][k] * E2M1(wq, n, k)
 *   xq u8 (M,K), ea u32 [K/128][M] (fp8_quant_mx), wq u8 (N, K/2),
 *   eb u32 [K/128][N] (fp8_quant_mxfp4), y bf16 bits (M,N); K % 128 == 0.
 *   The scaled matrix instruction takes W as an E2M1 operand and each lane's
 *   group scale; the K sum stays in its FP32 accumulator.  Accuracy: that of
 *   the FP8 instruction, as for fp8_gemm_nt_mx.  flags must be 0.
 */
fp8_status fp8_gemm_nt_mx_w4(const uint8_t* xq, const uint32_t* ea,
                             const uint8_t* wq, const uint32_t* eb, uint16_t* y,
                             int64_t M, int64_t N, int64_t K, uint32_t flags,
                             void* stream);

/*
 * The kernel instances a GEMM call would launch, computed on the host from
 * the shape and a compute-unit count (no device needed): the persistent tile
 * schedule of [DG] "统一块调度器与 rasterization" and the tile choice of
 * [DG] "非对齐块大小" (pick the tile whose count fills the machine's waves
 * best).
 *   layout   0 dense (fp8_gemm_nt), 1 contiguous, 2 masked (max_m as M)
 *   flags    FP8_FLAG_* of the call, plus FP8_PLAN_MX (fp8_gemm_nt_mx /
 *            fp8_gemm_nt_mx_w4) or FP8_PLAN_QOUT (fp8_gemm_nt_qout), dense only
 *   workspace_bytes  what an fp8_gemm_nt_ws call would pass
 * Masked plans count every expert's max_m rows (the kernel counts the valid
 * ones on the device), per expert.  A masked launch has one workgroup per
 * possible tile (grid = tiles per expert, times E at the call); every other
 * tile-kernel launch is persistent (grid = min(tiles, CUs)).
 */
#define FP8_PLAN_MX 0x100u
#define FP8_PLAN_QOUT 0x200u
typedef struct {
    int32_t exact;          /* 1: exact partials (FP16 instruction); 0: FP8 instruction */
    int32_t kernel;         /* 0: tile kernel; 1: decode kernel (M <= 32); 2: X-resident decode kernel;
                               3: exact decode kernel (M <= 64, X in chunks); 4: exact decode kernel
                               with X resident (M <= 64, short K ranges) */
    int32_t tile_m, tile_n; /* workgroup tile of the main launch (decode kernels: all M rows x tile_n columns) */
    int32_t waves;          /* waves per workgroup */
    int32_t grid;           /* workgroups of the main launch */
    int64_t tiles;          /* tiles of the main launch (decode kernels: workgroups) */
    int64_t main_rows;      /* rows [0, main_rows) in the main launch (contiguous); else M */
    int32_t tail_tile_m, tail_tile_n; /* tile of a second launch, or 0: contiguous, over rows
                               [main_rows, M); dense, over columns [main_cols, N) */
    int64_t tail_tiles;
    int32_t k_splits;       /* decode kernel: workgroups along K per tile */
    size_t workspace_bytes; /* workspace the split uses */
    int64_t main_cols;      /* columns [0, main_cols) in the main launch (dense); else N */
    int32_t paired;         /* contiguous, 1: three launches share the 128-row blocks, split on
                               the device from m_indices: the main launch takes 256-row tiles
                               over pairs of consecutive blocks of one expert, the middle launch
                               (mid_tile_m x mid_tile_n) and the tail launch the blocks left,
                               each in whole rounds of its tiles where a last partial round
                               would leave over half of the compute units idle; tiles,
                               mid_tiles and tail_tiles are then upper bounds, and main_rows M */
    int32_t mid_tile_m, mid_tile_n;
    int64_t mid_tiles;
} fp8_gemm_plan_t;
fp8_status fp8_gemm_plan(int32_t layout, int64_t M, int64_t N, int64_t K,
                         uint32_t flags, int32_t compute_units,
                         size_t workspace_bytes, fp8_gemm_plan_t* plan);

/* M alignment every expert segment of the contiguous layout must have
 * ([DG] "分组 GEMM 的两种布局": the alignment query).  Returns 128. */
int32_t fp8_get_mk_alignment_for_contiguous_layout(void);

/* Static description of a status code (never NULL). */
const char* fp8_status_string(fp8_status status);

#ifdef __cplusplus
}
#endif
#endif
