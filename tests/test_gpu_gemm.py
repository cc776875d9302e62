"""GPU dense block-scaled GEMM against the oracle.

Two accumulation paths are tested:
  * the default path: exact block partials (E4M3 widened to FP16, FP16 matrix
    instruction) -- held to the tolerance |y - ref| <= 8e-3 |ref| +
    1e-3 rms(ref) on every element of every input;
  * the opt-in FP8_FLAG_FAST_ACCUM path (FP8 matrix instruction): held to that
    tolerance on the headline workloads (every element, slow tests) and
    elsewhere to the tolerance or the bound of the measured FP8-MFMA
    truncation model, with a ceiling on the elements outside the tolerance.
Bit-exact where the result is exactly representable (layout probes, small
integers with power-of-two scales) on both paths.
"""
import ctypes

import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import (assert_close, assert_close_or_bounded, bf16_bits, bf16_to_f64,
                         check_guards, dev, fp8_mfma_error_bound, guarded, say)

pytestmark = pytest.mark.gpu

DEC = oracle.e4m3_decode(np.arange(256))
PATHS = [pytest.param(False, id="exact"), pytest.param(True, id="fast")]


def run_gemm(xq, sa, wq, sb, ue8m0=False, fast=False, guard=2048):
    M, K = xq.shape
    N = wq.shape[0]
    say(f"gemm_nt M={M} N={N} K={K} ue8m0={ue8m0} fast_accum={fast}")
    full, y = guarded((M, N), guard)
    fp8.gemm_nt(dev(xq), dev(sa), dev(wq), dev(sb), ue8m0=ue8m0, fast_accum=fast, out=y)
    torch.cuda.synchronize()
    check_guards(full, M * N, guard)
    return bf16_bits(y)


def check(y, xq, sa, wq, sb, ref, fast, ue8m0=False, what=""):
    """The tolerance on every element (default path), or the FP8-instruction
    bound with its ceiling (FP8_FLAG_FAST_ACCUM)."""
    if not fast:
        return assert_close(y, ref, what)
    bound = fp8_mfma_error_bound(xq, sa, wq, sb, ref, pow2=ue8m0)
    return assert_close_or_bounded(y, ref, bound, what)


def check_sampled(y, ref, xq, sa, wq, sb, mi, ni, fast, ue8m0=False, what=""):
    """As check, on the sampled elements (mi, ni) of a large output."""
    if not fast:
        return assert_close(y[mi, ni], ref, what)
    M, N = xq.shape[0], wq.shape[0]
    bound = fp8_mfma_error_bound(xq, sa, wq, sb, np.zeros((M, N)), pow2=ue8m0)[mi, ni] \
        + 2.0 ** -8 * np.abs(ref)
    return assert_close_or_bounded(y[mi, ni], ref, bound, what)


def unit_scales(M, N, K):
    return np.ones((K // 128, M), np.float32), np.ones(((N + 127) // 128, K // 128), np.float32)


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M,N,K", [(64, 96, 256), (200, 256, 384), (512, 1024, 256)])
def test_layout_probe_onehot_x(M, N, K, fast):
    """X row m is one-hot at k(m): Y[m, n] = W[n, k(m)] exactly."""
    rng = np.random.default_rng(M + N)
    km = (np.arange(M) * 37 + 11) % K
    xq = np.zeros((M, K), np.uint8)
    xq[np.arange(M), km] = 0x38          # 1.0
    wq = workloads.random_codes(rng, (N, K))
    sa, sb = unit_scales(M, N, K)
    y = run_gemm(xq, sa, wq, sb, fast=fast)
    assert np.array_equal(bf16_to_f64(y), DEC[wq][:, km].T)


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M,N,K", [(64, 96, 256), (200, 256, 384), (512, 1024, 256)])
def test_layout_probe_onehot_w(M, N, K, fast):
    """W row n is one-hot at k(n): Y[m, n] = X[m, k(n)] exactly."""
    rng = np.random.default_rng(M * N)
    kn = (np.arange(N) * 53 + 7) % K
    wq = np.zeros((N, K), np.uint8)
    wq[np.arange(N), kn] = 0x38
    xq = workloads.random_codes(rng, (M, K))
    sa, sb = unit_scales(M, N, K)
    y = run_gemm(xq, sa, wq, sb, fast=fast)
    assert np.array_equal(bf16_to_f64(y), DEC[xq][:, kn])


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M,N,K,ue8m0", [(64, 96, 256, False), (300, 384, 256, False),
                                         (130, 256, 256, True), (2048, 8192, 128, False)])
def test_exact_small_integers_pow2_scales(M, N, K, ue8m0, fast):
    """Codes in {0, +-1}, per-row and per-block power-of-two scales constant
    along K: every Y is 2^e times an integer of magnitude <= K = 256, exact in
    FP32 and BF16; the GPU must match bit for bit."""
    rng = np.random.default_rng(M + K)
    xq = rng.choice(np.array([0x00, 0x38, 0xB8], np.uint8), (M, K))
    wq = rng.choice(np.array([0x00, 0x38, 0xB8], np.uint8), (N, K))
    r = workloads.random_pow2(rng, M, -3, 3)
    c = workloads.random_pow2(rng, (N + 127) // 128, -3, 3)
    sa = np.ascontiguousarray(np.tile(r, (K // 128, 1)))
    sb = np.ascontiguousarray(np.tile(c[:, None], (1, K // 128)))
    ref = oracle.gemm_nt(xq, sa, wq, sb)
    y = run_gemm(xq, sa, wq, sb, ue8m0=ue8m0, fast=fast)
    assert np.array_equal(bf16_to_f64(y), ref)


@pytest.mark.parametrize("fast", PATHS)
def test_config1_parity_and_end_to_end(fast):
    """M=128, N=256, K=512 with 1% outliers x50: the tolerance on every element."""
    wl = workloads.config(1)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    ref = oracle.gemm_nt(xq, sa, wq, sb)
    y = run_gemm(xq, sa, wq, sb, fast=fast)
    assert_close(y, ref, "config 1")
    say("config 1 end to end")
    gxq, gsa = fp8.quant_1x128(dev(wl.x))
    gwq, gsb = fp8.quant_128x128(dev(wl.w))
    y2 = bf16_bits(fp8.gemm_nt(gxq, gsa, gwq, gsb, fast_accum=fast))
    assert np.array_equal(y2, y)


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M,N,K", [(1, 16, 128), (63, 96, 256), (65, 224, 384), (300, 300, 256),
                                   (257, 130, 128), (5, 50, 256), (64, 1536, 1536),
                                   (1000, 777, 640)])
def test_ragged_shapes(M, N, K, fast):
    wl = workloads.dense(M, N, K, seed=M * 7 + N, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    ref = oracle.gemm_nt(xq, sa, wq, sb)
    y = run_gemm(xq, sa, wq, sb, fast=fast)
    say(f"stats {check(y, xq, sa, wq, sb, ref, fast, what=f'{M}x{N}x{K}')}")


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M,N,K", [(96, 256, 512), (2048, 8192, 256)])
def test_ue8m0_paths(M, N, K, fast):
    wl = workloads.dense(M, N, K, seed=M + 3, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x, oracle.FLAG_UE8M0)
    wq, sb = oracle.quant_128x128(wl.w, oracle.FLAG_UE8M0)
    y = run_gemm(xq, sa, wq, sb, ue8m0=True, fast=fast)
    if M * N <= 1 << 16:
        ref = oracle.gemm_nt(xq, sa, wq, sb, oracle.FLAG_UE8M0)
        say(f"stats {check(y, xq, sa, wq, sb, ref, fast, ue8m0=True, what='ue8m0')}")
    else:
        rng = np.random.default_rng(1)
        mi, ni = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
        ref = oracle.gemm_nt_elems(xq, sa, wq, sb, mi, ni, oracle.FLAG_UE8M0)
        say(f"stats {check_sampled(y, ref, xq, sa, wq, sb, mi, ni, fast, True, 'ue8m0 sampled')}")


@pytest.mark.parametrize("fast", PATHS)
def test_large_tile_instance_sampled(fast):
    """A shape with >= 512 tiles of 256x128 takes the large-tile instance."""
    M, N, K = 2048, 8192, 384
    wl = workloads.dense(M, N, K, seed=9, outlier_frac=0.001, outlier_mult=100.0)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    y = run_gemm(xq, sa, wq, sb, fast=fast)
    rng = np.random.default_rng(2)
    mi, ni = rng.integers(0, M, 30000), rng.integers(0, N, 30000)
    mi = np.concatenate([mi, np.zeros(N, int), np.full(N, M - 1), np.arange(M), np.arange(M)])
    ni = np.concatenate([ni, np.arange(N), np.arange(N), np.zeros(M, int), np.full(M, N - 1)])
    ref = oracle.gemm_nt_elems(xq, sa, wq, sb, mi, ni)
    say(f"stats {check_sampled(y, ref, xq, sa, wq, sb, mi, ni, fast, what='large tiles')}")


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("ue8m0", [False, True])
def test_huge_tile_instance_ragged_sampled(ue8m0, fast):
    """At least one 256x256 tile per compute unit takes the 256x256 instance
    (both paths): here with a ragged last tile in M and N (N not a multiple of
    4) and an odd number of K blocks; every row and column of the ragged edges
    is checked."""
    M, N, K = 1900, 8102, 640
    flags = oracle.FLAG_UE8M0 if ue8m0 else 0
    wl = workloads.dense(M, N, K, seed=13, outlier_frac=0.001, outlier_mult=100.0)
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    y = run_gemm(xq, sa, wq, sb, ue8m0=ue8m0, fast=fast)
    rng = np.random.default_rng(3)
    mi, ni = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
    edge_m, edge_n = np.arange(1792, M), np.arange(7936, N)
    mi = np.concatenate([mi, np.repeat(edge_m, 16), rng.integers(0, M, 16 * len(edge_n)), np.full(N, M - 1)])
    ni = np.concatenate([ni, rng.integers(0, N, 16 * len(edge_m)), np.repeat(edge_n, 16), np.arange(N)])
    ref = oracle.gemm_nt_elems(xq, sa, wq, sb, mi, ni, flags)
    say(f"stats {check_sampled(y, ref, xq, sa, wq, sb, mi, ni, fast, ue8m0, '256x256 tiles, ragged edges')}")


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("ue8m0", [False, True])
def test_224_wide_tile_instance_ragged_sampled(ue8m0, fast):
    """Shapes that fill whole waves with 256x224 tiles but not with 256x256
    ones take the 256x224 instance on the FP8-instruction path, which holds X
    in registers and streams the W subtiles: here 10 x 32 tiles, the last n
    tile holding 106 columns that straddle two weight blocks, a ragged last m
    tile and an odd number of K blocks.  The default path splits the columns:
    [0, 6400) in 256x256 tiles, [6400, 7050) in 256x192 tiles whose last one
    holds 74 columns.  Every row and column of the ragged edges is checked."""
    M, N, K = 2500, 7050, 640
    flags = oracle.FLAG_UE8M0 if ue8m0 else 0
    wl = workloads.dense(M, N, K, seed=17, outlier_frac=0.001, outlier_mult=100.0)
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    y = run_gemm(xq, sa, wq, sb, ue8m0=ue8m0, fast=fast)
    rng = np.random.default_rng(5)
    mi, ni = rng.integers(0, M, 20000), rng.integers(0, N, 20000)
    edge_m, edge_n = np.arange(2304, M), np.arange(6944, N)
    mi = np.concatenate([mi, np.repeat(edge_m, 16), rng.integers(0, M, 16 * len(edge_n)), np.full(N, M - 1)])
    ni = np.concatenate([ni, rng.integers(0, N, 16 * len(edge_m)), np.repeat(edge_n, 16), np.arange(N)])
    ref = oracle.gemm_nt_elems(xq, sa, wq, sb, mi, ni, flags)
    say(f"stats {check_sampled(y, ref, xq, sa, wq, sb, mi, ni, fast, ue8m0, '256x224 tiles, ragged edges')}")


@pytest.mark.parametrize("ue8m0", [False, True])
@pytest.mark.parametrize("M,N,K", [(1, 48, 128), (16, 1000, 384), (17, 777, 640), (32, 130, 1536),
                                   (24, 4096, 896), (32, 3072, 1536), (30, 50, 128), (20, 2, 256),
                                   (32, 200, 7168), (8, 500, 2176), (32, 24576, 256), (9, 24700, 640),
                                   (33, 130, 1536), (64, 200, 896), (48, 24576, 256), (48, 1000, 1664),
                                   (40, 300, 128), (36, 97, 1408), (48, 200, 1792), (45, 4000, 1152),
                                   (64, 300, 1536), (50, 97, 128), (57, 1000, 640), (64, 24700, 1152),
                                   (49, 130, 1536), (64, 96, 256), (64, 300, 1792)])
@pytest.mark.parametrize("fast", PATHS)
def test_decode_instance(M, N, K, ue8m0, fast):
    """M <= 32 takes the decode kernel (one wave per 16 W rows over all of K,
    X and the scales in chunks of four K blocks): one and two 16-row subtiles
    of X, a single K block, partial last chunks (K = 384, 640, 896, 2176),
    many chunks (7168), K split over 2 to 8 workgroups per column tile when
    the tiles are fewer than the CUs (uneven chunk ranges at K = 2176), a grid
    of more than one workgroup per CU with a ragged last tile (N 24700), N
    edges inside a tile, waves wholly past N and tiles straddling a weight
    block.  33 <= M <= 48 with K <= 1664 takes the
    X-resident decode kernel (K groups of waves, a single K block, fewer
    blocks than K groups, the largest K, ragged N); 49 <= M <= 64 takes the
    64x96 tile of the main kernel (one K block, ragged N, an N edge inside a
    tile, a single tile), as do K = 1792 and above.  These are the
    FP8-instruction kernels (FP8_FLAG_FAST_ACCUM, with a workspace for the
    split).  The default path takes its exact decode kernel: with X resident
    in LDS for M <= 32, and split over K (a workspace comes with the call)
    when the 96-column tiles are fewer than the CUs, each range holding at
    most 24 K blocks (M <= 32) or 12 (M > 32), else with X in chunks; unsplit
    with M > 32 it takes the 64x96 tile.  Every element."""
    flags = oracle.FLAG_UE8M0 if ue8m0 else 0
    wl = workloads.dense(M, N, K, seed=M * 31 + N + K, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    ref = oracle.gemm_nt(xq, sa, wq, sb, flags)
    y = run_gemm(xq, sa, wq, sb, ue8m0=ue8m0, fast=fast)
    say(f"stats {check(y, xq, sa, wq, sb, ref, fast, ue8m0=ue8m0, what=f'decode {M}x{N}x{K}')}")


@pytest.mark.parametrize("ue8m0", [False, True])
@pytest.mark.parametrize("M,N,K", [(64, 4096, 7168), (32, 1000, 3200), (17, 777, 3328), (64, 130, 1664),
                                   (1, 200, 1792), (40, 24700, 2048)])
def test_exact_decode_without_workspace(M, N, K, ue8m0):
    """The default path through fp8_gemm_nt, which passes no workspace: for
    M <= 32 the exact decode kernel runs unsplit, X resident in LDS up to 24
    K blocks and streamed in chunks of four K blocks beyond (partial last
    chunks included); for 32 < M <= 64 the 64x96 tile of the main kernel.
    Every element."""
    L = fp8.load_library()
    flags = oracle.FLAG_UE8M0 if ue8m0 else 0
    plan = fp8.gemm_plan("dense", M, N, K, ue8m0=ue8m0)
    assert plan["kernel"] == ((4 if K // 128 <= 24 else 3) if M <= 32 else 0) and plan["k_splits"] == 1
    wl = workloads.dense(M, N, K, seed=M + N + K, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    a = [dev(t) for t in (xq, sa, wq, sb)]
    full, y = guarded((M, N))
    say(f"fp8_gemm_nt (no workspace) M={M} N={N} K={K} ue8m0={ue8m0} kernel={plan['kernel']}")
    st = L.fp8_gemm_nt(*[ctypes.c_void_p(t.data_ptr()) for t in a], ctypes.c_void_p(y.data_ptr()), M, N, K, flags,
                       ctypes.c_void_p(torch.cuda.current_stream().cuda_stream))
    assert st == 0
    torch.cuda.synchronize()
    check_guards(full, M * N)
    ref = oracle.gemm_nt(xq, sa, wq, sb, flags)
    say(f"stats {assert_close(bf16_bits(y), ref, f'no-workspace decode {M}x{N}x{K}')}")


def test_decode_instance_deterministic():
    """Repeated calls agree bit for bit, also when K is split over workgroups
    (FP8_FLAG_FAST_ACCUM, here 50 column tiles, 8 splits): the partial sums
    are added in split order."""
    wl = workloads.dense(32, 4800, 7168, seed=5, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    a = [dev(t) for t in (xq, sa, wq, sb)]
    say("decode determinism x10")
    first = bf16_bits(fp8.gemm_nt(*a, fast_accum=True))
    for _ in range(9):
        assert np.array_equal(bf16_bits(fp8.gemm_nt(*a, fast_accum=True)), first)


@pytest.mark.parametrize("fast", PATHS)
def test_deterministic_repeats(fast):
    wl = workloads.dense(300, 512, 1024, seed=77, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    a = [dev(t) for t in (xq, sa, wq, sb)]
    say(f"determinism x10 fast_accum={fast}")
    first = bf16_bits(fp8.gemm_nt(*a, fast_accum=fast))
    for _ in range(9):
        assert np.array_equal(bf16_bits(fp8.gemm_nt(*a, fast_accum=fast)), first)


@pytest.mark.slow
@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("cfg", [2, 3])
def test_full_size_dense_configs_every_element(cfg, fast):
    """The headline dense workloads: the tolerance on all M*N elements."""
    wl = workloads.config(cfg)
    say(f"config {cfg}: oracle quantization")
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    y = run_gemm(xq, sa, wq, sb, fast=fast)
    say(f"config {cfg}: oracle GEMM ({2 * xq.shape[0] * wq.shape[0] * xq.shape[1]:.3g} FLOP)")
    ref = oracle.gemm_nt(xq, sa, wq, sb)
    stats = assert_close(y, ref, f"config {cfg}")
    say(f"config {cfg} error stats: {stats}")


def _split_operands(seed, M=16, N=2112, K=7168):
    """A decode shape with few column tiles (K split over workgroups on the
    FP8-instruction path, given a workspace)."""
    wl = workloads.dense(M, N, K, seed=seed, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    return [dev(t) for t in (xq, sa, wq, sb)]


@pytest.mark.slow
@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("M", [16, 100])
def test_largest_k(M, fast):
    """K = 2^22, the largest K the library takes (its per-lane tile offsets
    are 32-bit): random finite codes and power-of-two scales.  M = 16 takes
    the 64x96 tile (default path) or the decode kernel with K split over
    workgroups (FP8 instruction), M = 100 a 128-row tile.  The first 32
    columns are checked against the oracle on every row."""
    N, K = 256, 1 << 22
    rng = np.random.default_rng(M)
    say(f"largest K: M={M} codes")
    xq = workloads.random_codes(rng, (M, K))
    wq = workloads.random_codes(rng, (N, K))
    sa = workloads.random_pow2(rng, (K // 128, M), -8, 0)
    sb = workloads.random_pow2(rng, (N // 128, K // 128), -8, 0)
    y = run_gemm(xq, sa, wq, sb, guard=256, fast=fast)
    say("largest K: oracle on 32 columns")
    ref = oracle.gemm_nt(xq, sa, wq[:32], sb[:1])
    say(f"stats {check(y[:, :32], xq, sa, wq[:32], sb[:1], ref, fast, what=f'K=2^22 M={M}')}")


def test_split_decode_workspace_and_streams():
    """FP8_FLAG_FAST_ACCUM split-K decode GEMMs through fp8_gemm_nt_ws: with the
    workspace (K split over 8 workgroups per tile) the result is within the
    model bound of the oracle and equal, bit for bit, on two streams at once
    (each call with its own workspace) to the default-stream result; without a
    workspace (fp8_gemm_nt) the GEMM runs unsplit, also within the bound."""
    wl = workloads.dense(16, 2112, 7168, seed=45, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    ref = oracle.gemm_nt(xq, sa, wq, sb)
    a = [dev(t) for t in (xq, sa, wq, sb)]
    nbytes = fp8.load_library().fp8_gemm_workspace_size(16, 2112, 7168, fp8.FLAG_FAST_ACCUM)
    assert nbytes == 8 * 16 * 2112 * 4, nbytes
    say("split decode: workspace vs none")
    split = bf16_bits(fp8.gemm_nt(*a, fast_accum=True))
    ws0 = torch.empty(0, dtype=torch.uint8, device="cuda")
    unsplit = bf16_bits(fp8.gemm_nt(*a, fast_accum=True, workspace=ws0))
    check(split, xq, sa, wq, sb, ref, True, what="split")
    check(unsplit, xq, sa, wq, sb, ref, True, what="unsplit")
    ops = [a, _split_operands(42)]
    base = [bf16_bits(fp8.gemm_nt(*o, fast_accum=True)) for o in ops]
    streams = [torch.cuda.Stream(), torch.cuda.Stream()]
    outs = [torch.empty((16, 2112), dtype=torch.bfloat16, device="cuda") for _ in ops]
    torch.cuda.synchronize()
    say("split decode: two streams, 10 rounds")
    for _ in range(10):
        for o, st, y in zip(ops, streams, outs):
            with torch.cuda.stream(st):
                fp8.gemm_nt(*o, fast_accum=True, out=y)
        torch.cuda.synchronize()
        for r, y in zip(base, outs):
            assert np.array_equal(bf16_bits(y), r)


@pytest.mark.parametrize("fast", PATHS)
def test_split_decode_graph_replays(fast):
    """A split-K decode GEMM (both paths, workspace from torch's graph pool)
    captured in a graph: every replay, with eager work and synchronizations
    between replays, equals the eager result bit for bit."""
    o = _split_operands(43)
    assert fp8.load_library().fp8_gemm_workspace_size(16, 2112, 7168, fp8.FLAG_FAST_ACCUM if fast else 0) > 0
    s = torch.cuda.Stream()
    y = torch.empty((16, 2112), dtype=torch.bfloat16, device="cuda")
    with torch.cuda.stream(s):
        fp8.gemm_nt(*o, fast_accum=fast, out=y)
    torch.cuda.synchronize()
    eager = bf16_bits(y)
    g = torch.cuda.CUDAGraph()
    say(f"split decode: capture fast_accum={fast}")
    with torch.cuda.graph(g, stream=s):
        fp8.gemm_nt(*o, fast_accum=fast, out=y)
    other = _split_operands(44)
    for i in range(4):
        y.zero_()
        g.replay()
        fp8.gemm_nt(*other, fast_accum=fast)   # eager work on the default stream between replays
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), eager), f"replay {i}"


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("ue8m0", [False, True])
@pytest.mark.parametrize("M,N,K", [(300, 384, 1024), (16, 1000, 1024), (64, 24700, 1024), (2048, 2048, 768)])
def test_zero_scale_blocks(M, N, K, ue8m0, fast):
    """A zero scale comes with all-zero codes in its group (the header's
    contract): such groups, in the middle of K and at its ends, of X rows and
    of W blocks, add nothing, on every kernel (main tiles, the decode
    kernels).  The default path keeps its accumulator in units of the
    current block's scale product and must skip the zero factor."""
    flags = oracle.FLAG_UE8M0 if ue8m0 else 0
    wl = workloads.dense(M, N, K, seed=M + N + 7, outlier_frac=0.01, outlier_mult=50.0)
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    rng = np.random.default_rng(M)
    KB = K // 128
    for kb in (0, KB // 2, KB - 1):
        rows = rng.choice(M, size=max(1, M // 3), replace=False)
        xq[rows, 128 * kb:128 * (kb + 1)] = 0
        sa[kb, rows] = 0.0
    nb = (N + 127) // 128
    for kb, b in ((1, 0), (KB - 1, nb - 1)):
        wq[128 * b:128 * (b + 1), 128 * kb:128 * (kb + 1)] = 0
        sb[b, kb] = 0.0
    ref = oracle.gemm_nt(xq, sa, wq, sb, flags)
    y = run_gemm(xq, sa, wq, sb, ue8m0=ue8m0, fast=fast)
    say(f"stats {check(y, xq, sa, wq, sb, ref, fast, ue8m0=ue8m0, what=f'zero scales {M}x{N}x{K}')}")
