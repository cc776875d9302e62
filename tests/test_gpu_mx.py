"""GPU MXFP8 path (E4M3 with one E8M0 scale per 1x32 group on both operands)
against the oracle.

The quantizer is bit-exact (codes and scale bytes; the library packs the
bytes into [K/128][rows] dwords, the oracle keeps them (rows, K/32)).  The GEMM runs the scaled
FP8 matrix instruction with each lane's own group scale and keeps the K sum in
its FP32 accumulator; on random data it is held to the tolerance
|y - ref| <= 8e-3 |ref| + 1e-3 rms(ref) on every compared element, and
bit-exact where the result is exactly representable.  (The instruction's
truncation of small products inside each group of 8 K -- the bound stated for
FP8_FLAG_FAST_ACCUM -- can exceed the tolerance on crafted cancellations; the
MX calls have no exact-partial path.)"""
import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import (assert_close, bf16_bits, bf16_to_f64, check_guards, dev,
                         guarded, host, say)

pytestmark = pytest.mark.gpu

DEC = oracle.e4m3_decode(np.arange(256))


def pack_scales(e: np.ndarray) -> np.ndarray:
    """The oracle's (R, K/32) scale bytes in the library's packed layout: int32
    [K/128][R] whose byte t of [kb][r] is group 4*kb + t of row r."""
    R, G = e.shape
    return np.ascontiguousarray(e.reshape(R, G // 4, 4).transpose(1, 0, 2)).view(np.int32).reshape(G // 4, R)


def unpack_scales(p: np.ndarray) -> np.ndarray:
    KB, R = p.shape
    return np.ascontiguousarray(p.view(np.uint8).reshape(KB, R, 4).transpose(1, 0, 2)).reshape(R, 4 * KB)


def run_mx(xq, ea, wq, eb, guard=2048):
    M, K = xq.shape
    N = wq.shape[0]
    say(f"gemm_nt_mx M={M} N={N} K={K}")
    full, y = guarded((M, N), guard)
    fp8.gemm_nt_mx(dev(xq), dev(pack_scales(ea)), dev(wq), dev(pack_scales(eb)), out=y)
    torch.cuda.synchronize()
    check_guards(full, M * N, guard)
    return bf16_bits(y)


@pytest.mark.parametrize("R,K", [(128, 512), (1, 128), (300, 1024), (77, 384), (9, 7168),
                                 # a row of 32-group units plus a short one
                                 (33, 1152), (5, 2176)])
def test_quant_mx_bitexact(R, K):
    wl = workloads.dense(R, 1, K, seed=300 + R, outlier_frac=0.01, outlier_mult=50.0)
    q_ref, e_ref = oracle.quant_mx(wl.x)
    say(f"quant_mx R={R} K={K}")
    q, e = fp8.quant_mx(dev(wl.x))
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref)
    assert np.array_equal(unpack_scales(host(e)), e_ref)


def test_quant_mx_zero_and_tiny_groups():
    x = np.zeros((3, 256), np.float32)
    x[1, 32:64] = np.float32(1e-7)
    x[2, :] = -0.0
    x[2, 100] = 3.0
    q_ref, e_ref = oracle.quant_mx(x)
    q, e = fp8.quant_mx(dev(x))
    torch.cuda.synchronize()
    assert np.array_equal(host(q), q_ref) and np.array_equal(unpack_scales(host(e)), e_ref)


@pytest.mark.parametrize("M,N,K", [(128, 256, 512), (1, 96, 128), (64, 288, 1536), (200, 300, 384),
                                   (257, 129, 256), (600, 1000, 1024)])
def test_gemm_mx_every_element(M, N, K):
    """Covers the decode (64x96), 128x128 and 256x128 instances, ragged M and
    N edges and single rows."""
    wl = workloads.dense(M, N, K, seed=M + 7 * N, outlier_frac=0.01, outlier_mult=50.0)
    xq, ea = oracle.quant_mx(wl.x)
    wq, eb = oracle.quant_mx(wl.w)
    y = run_mx(xq, ea, wq, eb)
    ref = oracle.gemm_mx(xq, ea, wq, eb)
    assert_close(y, ref, f"mx {M}x{N}x{K}")


def test_gemm_mx_integer_products_are_exact():
    """Integer-valued codes with unit and power-of-two scales that cancel
    (2^3 * 2^-3): every product and partial sum is a small integer, so the
    BF16 result is exactly the oracle's."""
    rng = np.random.default_rng(9)
    M, N, K = 96, 160, 256
    small = np.array([0x00, 0x38, 0x40, 0xB8, 0xC0], np.uint8)   # 0, 1, 2, -1, -2
    xq = rng.choice(small, (M, K)).astype(np.uint8)
    wq = rng.choice(small, (N, K)).astype(np.uint8)
    ea = np.full((M, K // 32), 130, np.uint8)
    eb = np.full((N, K // 32), 124, np.uint8)
    y = run_mx(xq, ea, wq, eb)
    ref = oracle.gemm_mx(xq, ea, wq, eb)
    assert np.all(np.abs(ref) <= 256)
    assert np.array_equal(bf16_to_f64(y), ref)


@pytest.mark.parametrize("M,N,K", [(2500, 7050, 640), (1900, 8102, 640)])
def test_gemm_mx_large_tiles_sampled(M, N, K):
    """The 256x224 (streamed W) and 256x256 instances, ragged last tiles in M
    and N, an odd number of K blocks; every row and column of the ragged
    edges is checked."""
    wl = workloads.dense(M, N, K, seed=M + N, outlier_frac=0.001, outlier_mult=100.0)
    xq, ea = oracle.quant_mx(wl.x)
    wq, eb = oracle.quant_mx(wl.w)
    y = run_mx(xq, ea, wq, eb)
    rng = np.random.default_rng(6)
    em = np.arange(M - M % 256 if M % 256 else M - 256, M)
    en = np.arange(N - 200, N)
    mi = np.concatenate([rng.integers(0, M, 20000), np.repeat(em, 8), rng.integers(0, M, 8 * len(en))])
    ni = np.concatenate([rng.integers(0, N, 20000), rng.integers(0, N, 8 * len(em)), np.repeat(en, 8)])
    ref = oracle.gemm_mx_elems(xq, ea, wq, eb, mi, ni)
    assert_close(y[mi, ni], ref, f"mx {M}x{N}x{K} sampled")


def test_gemm_mx_end_to_end_from_fp32():
    """GPU quantizer then GPU GEMM, against the oracle on the same FP32 input."""
    wl = workloads.dense(256, 512, 1024, seed=21, outlier_frac=0.001, outlier_mult=100.0)
    x, w = dev(wl.x), dev(wl.w)
    xq, ea = fp8.quant_mx(x)
    wq, eb = fp8.quant_mx(w)
    y = fp8.gemm_nt_mx(xq, ea, wq, eb)
    torch.cuda.synchronize()
    rx, rea = oracle.quant_mx(wl.x)
    rw, reb = oracle.quant_mx(wl.w)
    assert np.array_equal(host(xq), rx) and np.array_equal(unpack_scales(host(ea)), rea)
    assert np.array_equal(host(wq), rw) and np.array_equal(unpack_scales(host(eb)), reb)
    ref = oracle.gemm_mx(rx, rea, rw, reb)
    assert_close(bf16_bits(y), ref, "mx e2e")


def sample_with_edges(M, N, seed, n=4000):
    rng = np.random.default_rng(seed)
    mi = np.concatenate([rng.integers(0, M, n), np.zeros(256, int), np.full(256, M - 1), rng.integers(0, M, 512)])
    ni = np.concatenate([rng.integers(0, N, n), rng.integers(0, N, 512), np.zeros(256, int), np.full(256, N - 1)])
    return mi, ni


@pytest.mark.slow
def test_mx_full_size_config3_every_element():
    """The MXFP8 variant of the decode workload (64x24576x1536), as bench.py --mx
    times it: GPU quantizers bit-exact, GEMM within the tolerance on every element."""
    wl = workloads.config(3)
    say("mx config 3: quantizers")
    xq, ea = fp8.quant_mx(dev(wl.x))
    wq, eb = fp8.quant_mx(dev(wl.w))
    rx, rea = oracle.quant_mx(wl.x)
    rw, reb = oracle.quant_mx(wl.w)
    assert np.array_equal(host(xq), rx) and np.array_equal(unpack_scales(host(ea)), rea)
    assert np.array_equal(host(wq), rw) and np.array_equal(unpack_scales(host(eb)), reb)
    y = run_mx(rx, rea, rw, reb)
    say("mx config 3: oracle GEMM")
    ref = oracle.gemm_mx(rx, rea, rw, reb)
    assert_close(y, ref, "mx config 3")


@pytest.mark.slow
def test_mx_full_size_config2_sampled():
    """The MXFP8 variant of the prefill workload (4096x7168x7168), the 256x224
    instance that bench.py --mx times: quantizers bit-exact, GEMM on 5000
    sampled elements including the first and last rows and columns."""
    wl = workloads.config(2)
    say("mx config 2: oracle quantizers")
    rx, rea = oracle.quant_mx(wl.x)
    rw, reb = oracle.quant_mx(wl.w)
    xq, ea = fp8.quant_mx(dev(wl.x))
    wq, eb = fp8.quant_mx(dev(wl.w))
    assert np.array_equal(host(xq), rx) and np.array_equal(unpack_scales(host(ea)), rea)
    assert np.array_equal(host(wq), rw) and np.array_equal(unpack_scales(host(eb)), reb)
    y = run_mx(rx, rea, rw, reb)
    M, N = y.shape
    mi, ni = sample_with_edges(M, N, 11)
    ref = oracle.gemm_mx_elems(rx, rea, rw, reb, mi, ni)
    assert_close(y[mi, ni], ref, "mx config 2 sampled")
