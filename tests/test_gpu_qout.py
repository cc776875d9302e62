"""GEMM with the output quantized in its epilogue for the next GEMM
(fp8_gemm_nt_qout: E4M3 codes + 1x128 scales along N) against the oracle.

Where the FP32 accumulator is exact (integer-valued products, power-of-two
scales, small sums) the codes and scales must be bit-identical to the 1x128
oracle quantizer applied to the exact product, on both accumulation paths.
Elsewhere the accumulator may differ from the exact product by a bound B --
FP32 accumulation on the default path (exact partials), the FP8-MFMA model
bound with FP8_FLAG_FAST_ACCUM -- so each group's scale must lie between
fl32((A-B)/448) and fl32((A+B)/448), A the exact group maximum, and each
decoded value within half an E4M3 step of the exact one plus B."""
import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import bf16_bits, bf16_to_f64, dev, fp8_mfma_error_bound, host, say

pytestmark = pytest.mark.gpu

DEC = oracle.e4m3_decode(np.arange(256))
PATHS = [pytest.param(False, id="exact"), pytest.param(True, id="fast")]


def accumulation_bound(xq, sa, wq, sb, fast, pow2):
    """Per-element bound on |accumulator - exact product|: the FP8-MFMA model
    (fast), or 2^-18 of the sum of |scaled products| (exact partials summed in
    FP32: at most a few dozen roundings of 2^-24 each along K)."""
    if fast:
        return fp8_mfma_error_bound(xq, sa, wq, sb, np.zeros((xq.shape[0], wq.shape[0])), pow2=pow2)
    M, K = xq.shape
    N = wq.shape[0]
    sx = np.repeat(sa.astype(np.float64).T, 128, axis=1)
    sw = np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    return 2.0 ** -18 * ((np.abs(DEC[xq]) * sx) @ (np.abs(DEC[wq]) * sw).T)


def integer_case(rng, M, N, K):
    small = np.array([0x00, 0x38, 0x40, 0x44, 0xB8, 0xC0, 0xC4], np.uint8)   # 0, ±1, ±2, ±3
    xq = rng.choice(small, (M, K)).astype(np.uint8)
    wq = rng.choice(small, (N, K)).astype(np.uint8)
    sa = np.exp2(rng.integers(-2, 3, (K // 128, M))).astype(np.float32)
    sb = np.exp2(rng.integers(-2, 3, ((N + 127) // 128, K // 128))).astype(np.float32)
    return xq, sa, wq, sb


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M,N,K,ue8m0", [(96, 256, 256, False), (300, 384, 512, False),
                                         (300, 384, 512, True), (2048, 8192, 256, False)])
def test_qout_bitexact_when_the_accumulator_is_exact(M, N, K, ue8m0, fast):
    rng = np.random.default_rng(M + N)
    xq, sa, wq, sb = integer_case(rng, M, N, K)
    flags = oracle.FLAG_UE8M0 if ue8m0 else 0
    say(f"gemm_nt_qout M={M} N={N} K={K} ue8m0={ue8m0} fast_accum={fast}")
    yq, sy = fp8.gemm_nt_qout(dev(xq), dev(sa), dev(wq), dev(sb), ue8m0=ue8m0, fast_accum=fast)
    torch.cuda.synchronize()
    y = oracle.gemm_nt(xq, sa, wq, sb, flags)
    assert np.all(np.abs(y) < 2 ** 24) and np.array_equal(y.astype(np.float32), y)   # exact in FP32
    q_ref, s_ref = oracle.quant_1x128(y.astype(np.float32), flags)
    assert np.array_equal(host(sy).view(np.uint32), s_ref.view(np.uint32))
    assert np.array_equal(host(yq), q_ref)


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M,N,K,ue8m0", [(200, 512, 1024, False), (256, 1024, 2048, True),
                                         (1024, 2048, 512, False)])
def test_qout_within_quantization_and_accumulation_bounds(M, N, K, ue8m0, fast):
    wl = workloads.dense(M, N, K, seed=M + K, outlier_frac=0.001, outlier_mult=100.0)
    flags = oracle.FLAG_UE8M0 if ue8m0 else 0
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    say(f"gemm_nt_qout M={M} N={N} K={K} ue8m0={ue8m0} fast_accum={fast}")
    yq, sy = fp8.gemm_nt_qout(dev(xq), dev(sa), dev(wq), dev(sb), ue8m0=ue8m0, fast_accum=fast)
    torch.cuda.synchronize()
    yq, sy = host(yq), host(sy)
    y = oracle.gemm_nt(xq, sa, wq, sb, flags)
    b = accumulation_bound(xq, sa, wq, sb, fast, ue8m0)
    G = N // 128
    A = np.abs(y).reshape(M, G, 128).max(axis=2)                              # exact group maxima
    Bg = b.reshape(M, G, 128).max(axis=2)

    def scale(a):
        s = (np.maximum(a, 1e-4).astype(np.float32) / np.float32(448.0)).astype(np.float32)
        if ue8m0:
            s = np.exp2(np.ceil(np.log2(s.astype(np.float64)))).astype(np.float32)
        return s
    lo, hi = scale(np.maximum(A - Bg, 0)), scale(A + Bg)
    s = sy.T                                                                  # (M, G)
    assert np.all((s >= lo * (1 - 2 ** -23)) & (s <= hi * (1 + 2 ** -23)))
    srow = np.repeat(s, 128, axis=1).astype(np.float64)
    d = DEC[yq] * srow
    allowed = 2.0 ** -4 * (np.abs(y) + b) + 2.0 ** -10 * srow + b
    assert np.all(np.abs(d - y) <= allowed)


@pytest.mark.parametrize("fast", PATHS)
def test_qout_feeds_the_next_gemm(fast):
    """X -> GEMM with quantized output -> its (yq, sy) as the next GEMM's
    activations, bit-exact end to end where every accumulator is exact."""
    rng = np.random.default_rng(5)
    M, N1, K, N2 = 128, 256, 384, 384
    xq, sa, w1, s1 = integer_case(rng, M, N1, K)
    _, _, w2, s2 = integer_case(rng, 1, N2, N1)
    say(f"chained gemm_nt_qout + gemm_nt fast_accum={fast}")
    yq, sy = fp8.gemm_nt_qout(dev(xq), dev(sa), dev(w1), dev(s1), fast_accum=fast)
    y2 = fp8.gemm_nt(yq, sy, dev(w2), dev(s2), fast_accum=fast)
    torch.cuda.synchronize()
    y1 = oracle.gemm_nt(xq, sa, w1, s1)
    q1, t1 = oracle.quant_1x128(y1.astype(np.float32))
    ref = oracle.gemm_nt(q1, t1, w2, s2)
    got = bf16_to_f64(bf16_bits(y2))
    rms = np.sqrt(np.mean(ref ** 2))
    assert np.all(np.abs(got - ref) <= 8e-3 * np.abs(ref) + 1e-3 * rms)
