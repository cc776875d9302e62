"""Accumulation precision of the FP8 matrix instruction and the promotion
interval (how many K blocks may be summed before scaling), measured through
the public entry points.

DeepGEMM page, section "细粒度缩放在 GEMM 层面引爆的两个问题": the FP8 tensor
cores of H800 accumulate with limited precision, which is why partials are
promoted into FP32 every 128 K.  On gfx950 the FP8 instruction drops low bits
of small products within each group of 8 consecutive K (the measured model in
gpu_helpers.fp8_mfma_error_bound), while its accumulator input C is added in
FP32.  Consequences tested here:
  * promoting every 128-K block by VALU FMA and accumulating the whole K in
    the scaled instruction's accumulator give bit-identical results on
    power-of-two scales: the longer interval costs no precision;
  * exact partials (the default path) give correctly rounded BF16 for almost
    every element, the FP8 instruction (FP8_FLAG_FAST_ACCUM) for most;
  * a crafted 8-group shows the truncation itself, and that the default path
    does not truncate."""
import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import bf16_bits, bf16_to_f64, dev, say

pytestmark = pytest.mark.gpu


def bf16_rne(v: np.ndarray) -> np.ndarray:
    """The exact values rounded once to BF16 (torch's RNE conversion of the
    FP32 rounding; FP32 then BF16 is a double rounding only for values within
    2^-24 relative of a BF16 tie, which the tolerance below absorbs)."""
    t = torch.from_numpy(v.astype(np.float32)).to(torch.bfloat16)
    return bf16_to_f64(t.view(torch.int16).numpy().view(np.uint16))


@pytest.mark.parametrize("M,N,K,outliers", [(256, 512, 7168, 0.001), (256, 512, 7168, 0.0),
                                            (128, 256, 28672, 0.001)])
def test_promotion_interval_128_equals_whole_k_on_pow2_scales(M, N, K, outliers):
    wl = workloads.dense(M, N, K, seed=K + M, outlier_frac=outliers, outlier_mult=100.0)
    xq, sa = oracle.quant_1x128(wl.x, oracle.FLAG_UE8M0)
    wq, sb = oracle.quant_128x128(wl.w, oracle.FLAG_UE8M0)
    a = [dev(t) for t in (xq, sa, wq, sb)]
    say(f"promotion interval M={M} N={N} K={K}")
    every_block = bf16_bits(fp8.gemm_nt(*a, fast_accum=True))              # zero-C FP8 partial + FP32 FMA per 128 K
    whole_k = bf16_bits(fp8.gemm_nt(*a, ue8m0=True, fast_accum=True))      # scaled instruction, K in its accumulator
    precise = bf16_bits(fp8.gemm_nt(*a))                                   # default: exact partials
    precise_pow2 = bf16_bits(fp8.gemm_nt(*a, ue8m0=True))                  # ... with exponent-shift promotion
    assert np.array_equal(every_block, whole_k)
    ref = oracle.gemm_nt(xq, sa, wq, sb, oracle.FLAG_UE8M0)
    rn = bf16_rne(ref)
    frac_precise = np.mean(bf16_to_f64(precise) == rn)
    assert np.mean(bf16_to_f64(precise_pow2) == rn) >= 0.999
    frac_fp8 = np.mean(bf16_to_f64(every_block) == rn)
    say(f"correctly rounded: precise {frac_precise:.4f}, fp8 {frac_fp8:.4f}")
    assert frac_precise >= 0.999          # measured 0.9998-0.9999
    assert 0.9 <= frac_fp8 < frac_precise  # measured 0.958-0.988


def test_fp8_instruction_truncates_small_products_in_a_group():
    """One 8-group holding 16*16 = 256 and seven products 0.125*0.125 = 2^-6;
    the next group holds -256.  Exact: 7 * 2^-6 = 0.109375.  In the measured
    model each product of a group is truncated toward zero to a multiple of
    2^(E-13), 2^E <= 256 being the group's largest: 2^-5 > 2^-6, so the seven
    vanish and the FP8-instruction paths (FP8_FLAG_FAST_ACCUM) return 0.  The
    default path's exact partials keep them, with FP32 or power-of-two scales."""
    K = 128
    xq = np.zeros((1, K), np.uint8)
    wq = np.zeros((16, K), np.uint8)
    xq[0, 0] = wq[0, 0] = 0x58            # 16
    xq[0, 1:8] = wq[0, 1:8] = 0x20        # 0.125
    xq[0, 8], wq[0, 8] = 0x58, 0xD8       # 16 * -16
    sa = np.ones((1, 1), np.float32)
    sb = np.ones((1, 1), np.float32)
    assert oracle.gemm_nt(xq, sa, wq, sb)[0, 0] == 0.109375
    a = [dev(t) for t in (xq, sa, wq, sb)]
    y = {k: bf16_to_f64(bf16_bits(fp8.gemm_nt(*a, **kw)))[0, 0]
         for k, kw in (("fp8", {"fast_accum": True}), ("fp8_ue8m0", {"ue8m0": True, "fast_accum": True}),
                       ("exact", {}), ("exact_ue8m0", {"ue8m0": True}))}
    assert y["exact"] == 0.109375 and y["exact_ue8m0"] == 0.109375
    assert y["fp8"] == 0.0 and y["fp8_ue8m0"] == 0.0
