"""GPU MXFP4-weight path (E2M1 weights, one E8M0 scale per 1x32 group; MXFP8
activations) against the oracle.

The weight quantizer is bit-exact (nibbles and scale bytes; the library packs
the scale bytes into [K/128][rows] dwords).  The GEMM runs the scaled matrix
instruction with an E2M1 A operand; on random data it is held to the
tolerance |y - ref| <= 8e-3 |ref| + 1e-3 rms(ref) on every compared element,
and bit-exact where the result is exactly representable."""
import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import assert_close, bf16_bits, bf16_to_f64, check_guards, dev, guarded, host, say
from test_gpu_mx import pack_scales, unpack_scales

pytestmark = pytest.mark.gpu

DEC8 = oracle.e4m3_decode(np.arange(256))
DEC4 = oracle.e2m1_decode(np.arange(16))


def unpack_nibbles(q):
    return np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1)


def run_w4(xq, ea, wq, eb, guard=2048):
    M, K = xq.shape
    N = wq.shape[0]
    say(f"gemm_nt_mx_w4 M={M} N={N} K={K}")
    full, y = guarded((M, N), guard)
    fp8.gemm_nt_mx_w4(dev(xq), dev(pack_scales(ea)), dev(wq), dev(pack_scales(eb)), out=y)
    torch.cuda.synchronize()
    check_guards(full, M * N, guard)
    return bf16_bits(y)


@pytest.mark.parametrize("R,K", [(96, 512), (1, 128), (300, 1024), (9, 7168), (33, 1152), (5, 2176)])
def test_quant_mxfp4_bitexact(R, K):
    wl = workloads.dense(1, R, K, seed=400 + R, outlier_frac=0.01, outlier_mult=50.0)
    q_ref, e_ref = oracle.quant_mxfp4(wl.w)
    say(f"quant_mxfp4 R={R} K={K}")
    q, e = fp8.quant_mxfp4(dev(wl.w))
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(unpack_scales(host(e)), e_ref)


def test_quant_mxfp4_ties_signs_and_zero_groups():
    """Every E2M1 midpoint (a tie) and its neighbours, with both signs, in
    groups whose scale is 1 (amax 6); a zero group; a -0 entry."""
    mags = DEC4[:8]
    mids = (mags[:-1] + mags[1:]) / 2
    vals = np.concatenate([mids, np.nextafter(mids.astype(np.float32), np.float32(0)),
                           np.nextafter(mids.astype(np.float32), np.float32(7)), mags]).astype(np.float32)
    row = np.zeros(256, np.float32)
    for g in range(8):
        row[32 * g] = 6.0                       # scale 1 for the group
        chunk = vals[(31 * g) % len(vals):][:31]
        row[32 * g + 1:32 * g + 1 + len(chunk)] = chunk * (1 if g % 2 == 0 else -1)
    x = np.stack([row, np.zeros(256, np.float32), -row])
    x[1, 5] = -0.0
    q_ref, e_ref = oracle.quant_mxfp4(x)
    q, e = fp8.quant_mxfp4(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref) and np.array_equal(unpack_scales(host(e)), e_ref)


@pytest.mark.parametrize("M,N,K", [(64, 288, 1536), (128, 256, 512), (1, 96, 128), (200, 300, 384),
                                   (257, 129, 256), (600, 1000, 1024)])
def test_gemm_mx_w4_every_element(M, N, K):
    wl = workloads.dense(M, N, K, seed=M + 3 * N, outlier_frac=0.01, outlier_mult=50.0)
    xq, ea = oracle.quant_mx(wl.x)
    wq, eb = oracle.quant_mxfp4(wl.w)
    y = run_w4(xq, ea, wq, eb)
    ref = oracle.gemm_mx_w4(xq, ea, wq, eb)
    assert_close(y, ref, f"w4 {M}x{N}x{K}")


def test_gemm_mx_w4_integer_products_are_exact():
    rng = np.random.default_rng(10)
    M, N, K = 96, 160, 256
    xq = rng.choice(np.array([0x00, 0x38, 0x40, 0xB8, 0xC0], np.uint8), (M, K)).astype(np.uint8)
    nib = rng.choice(np.array([0, 2, 4, 10, 12], np.uint8), (N, K))            # 0, 1, 2, -1, -2
    wq = (nib[:, 0::2] | (nib[:, 1::2] << 4)).astype(np.uint8)
    ea = np.full((M, K // 32), 129, np.uint8)
    eb = np.full((N, K // 32), 125, np.uint8)
    y = run_w4(xq, ea, wq, eb)
    ref = oracle.gemm_mx_w4(xq, ea, wq, eb)
    assert np.all(np.abs(ref) <= 256)
    assert np.array_equal(bf16_to_f64(y), ref)


@pytest.mark.parametrize("M,N,K", [(2500, 7050, 640), (1900, 8102, 640)])
def test_gemm_mx_w4_large_tiles_sampled(M, N, K):
    wl = workloads.dense(M, N, K, seed=M + N + 1, outlier_frac=0.001, outlier_mult=100.0)
    xq, ea = oracle.quant_mx(wl.x)
    wq, eb = oracle.quant_mxfp4(wl.w)
    y = run_w4(xq, ea, wq, eb)
    rng = np.random.default_rng(7)
    em = np.arange(M - (M % 256 if M % 256 else 256), M)
    en = np.arange(N - 200, N)
    mi = np.concatenate([rng.integers(0, M, 20000), np.repeat(em, 8), rng.integers(0, M, 8 * len(en))])
    ni = np.concatenate([rng.integers(0, N, 20000), rng.integers(0, N, 8 * len(em)), np.repeat(en, 8)])
    ref = oracle.gemm_mx_w4_elems(xq, ea, wq, eb, mi, ni)
    assert_close(y[mi, ni], ref, f"w4 {M}x{N}x{K} sampled")


def test_gemm_mx_w4_end_to_end_from_fp32():
    wl = workloads.dense(256, 512, 1024, seed=23, outlier_frac=0.001, outlier_mult=100.0)
    xq, ea = fp8.quant_mx(dev(wl.x))
    wq, eb = fp8.quant_mxfp4(dev(wl.w))
    y = fp8.gemm_nt_mx_w4(xq, ea, wq, eb)
    torch.cuda.synchronize()
    rx, rea = oracle.quant_mx(wl.x)
    rw, reb = oracle.quant_mxfp4(wl.w)
    assert np.array_equal(host(xq), rx) and np.array_equal(unpack_scales(host(ea)), rea)
    assert np.array_equal(host(wq), rw) and np.array_equal(unpack_scales(host(eb)), reb)
    ref = oracle.gemm_mx_w4(rx, rea, rw, reb)
    assert_close(bf16_bits(y), ref, "w4 e2e")


@pytest.mark.slow
def test_w4_full_size_config3_every_element():
    """MXFP8 activations x MXFP4 weights on the decode workload (64x24576x1536),
    as bench.py --w4 times it: GPU quantizers bit-exact, GEMM within the
    tolerance on every element."""
    wl = workloads.config(3)
    say("w4 config 3: quantizers")
    xq, ea = fp8.quant_mx(dev(wl.x))
    wq, eb = fp8.quant_mxfp4(dev(wl.w))
    rx, rea = oracle.quant_mx(wl.x)
    rw, reb = oracle.quant_mxfp4(wl.w)
    assert np.array_equal(host(xq), rx) and np.array_equal(unpack_scales(host(ea)), rea)
    assert np.array_equal(host(wq), rw) and np.array_equal(unpack_scales(host(eb)), reb)
    y = run_w4(rx, rea, rw, reb)
    say("w4 config 3: oracle GEMM")
    ref = oracle.gemm_mx_w4(rx, rea, rw, reb)
    assert_close(y, ref, "w4 config 3")


@pytest.mark.slow
def test_w4_full_size_config2_sampled():
    """MXFP8 x MXFP4 on the prefill workload (4096x7168x7168), the 256x224
    instance bench.py --w4 times: quantizers bit-exact, GEMM on 5000 sampled
    elements including the first and last rows and columns."""
    from test_gpu_mx import sample_with_edges
    wl = workloads.config(2)
    say("w4 config 2: oracle quantizers")
    rx, rea = oracle.quant_mx(wl.x)
    rw, reb = oracle.quant_mxfp4(wl.w)
    xq, ea = fp8.quant_mx(dev(wl.x))
    wq, eb = fp8.quant_mxfp4(dev(wl.w))
    assert np.array_equal(host(xq), rx) and np.array_equal(unpack_scales(host(ea)), rea)
    assert np.array_equal(host(wq), rw) and np.array_equal(unpack_scales(host(eb)), reb)
    y = run_w4(rx, rea, rw, reb)
    M, N = y.shape
    mi, ni = sample_with_edges(M, N, 13)
    ref = oracle.gemm_mx_w4_elems(rx, rea, rw, reb, mi, ni)
    assert_close(y[mi, ni], ref, "w4 config 2 sampled")
