"""Pins for the oracle's block-scaled GEMM (CPU only).

Each test ties the oracle to something other than its own formula:
  * unit scales / row-and-column-factorised scales reduce the method to a
    plain matrix product, computed here by numpy's library matmul (exact,
    because every sum of decoded E4M3 products is a short multiple of 2^-18);
  * integer codes with unit scales against an int64 library matmul;
  * quantize-then-GEMM of real data against the FP64 product of the original
    FP32 matrices, within the error bound that the quantizer pins establish;
  * invariance under a joint permutation of K blocks (with their scales).
A transposed operand, a wrong scale index or a dropped block fails at least
one of them.
"""
import numpy as np
import pytest

import oracle
import workloads

DEC = oracle.e4m3_decode(np.arange(256))


def _codes(rng, shape):
    return workloads.random_codes(rng, shape)


def test_unit_scales_equal_library_matmul_exactly():
    rng = np.random.default_rng(21)
    M, N, K = 37, 53, 1024
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones(((N + 127) // 128, K // 128), np.float32)
    y = oracle.gemm_nt(xq, sa, wq, sb)
    ref = DEC[xq] @ DEC[wq].T
    assert np.array_equal(y, ref)


def test_integer_partials_against_int64_matmul():
    rng = np.random.default_rng(22)
    M, N, K = 16, 24, 512
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    ia = (DEC[xq] * 512).astype(np.int64)      # every E4M3 value is j * 2^-9
    ib = (DEC[wq] * 512).astype(np.int64)
    assert np.array_equal(ia / 512.0, DEC[xq])
    sa = np.ones((K // 128, M), np.float32)
    sb = np.ones((1, K // 128), np.float32)
    y = oracle.gemm_nt(xq, sa, wq, sb)
    assert np.array_equal(y * 2.0 ** 18, (ia @ ib.T).astype(np.float64))


def test_row_and_block_column_scales_factorise():
    """sa[kb][m] = r_m and sb[nb][kb] = c_nb: Y = diag(r) (Xd Wd^T) diag(c)."""
    rng = np.random.default_rng(23)
    M, N, K = 40, 300, 384
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    r = workloads.random_pow2(rng, M)
    c = workloads.random_pow2(rng, 3)
    sa = np.tile(r, (K // 128, 1))
    sb = np.tile(c[:, None], (1, K // 128))
    y = oracle.gemm_nt(xq, sa, wq, sb)
    cn = np.repeat(c, 128)[:N].astype(np.float64)
    ref = (r.astype(np.float64)[:, None] * (DEC[xq] @ DEC[wq].T)) * cn[None, :]
    assert np.array_equal(y, ref)


def test_kblock_scales_against_prescaled_matmul():
    """Scales varying along K: matches the library matmul of element-wise
    dequantized matrices within binary64 rounding."""
    rng = np.random.default_rng(24)
    M, N, K = 20, 150, 768
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = rng.uniform(0.01, 3, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.01, 3, (2, K // 128)).astype(np.float32)
    y = oracle.gemm_nt(xq, sa, wq, sb)
    xd = DEC[xq] * np.repeat(sa.T.astype(np.float64), 128, axis=1)
    wd = DEC[wq] * np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    ref = xd @ wd.T
    mag = np.abs(xd) @ np.abs(wd).T
    assert np.all(np.abs(y - ref) <= 1e-13 * mag + 1e-300)


def test_quantized_gemm_close_to_unquantized_product():
    """End to end on data: |Y - X W^T| is bounded by the per-element
    quantization errors that the quantizer pins establish."""
    wl = workloads.dense(64, 200, 512, seed=25, outlier_frac=0.01, outlier_mult=50.0)
    x, w = wl.x.astype(np.float64), wl.w.astype(np.float64)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    y = oracle.gemm_nt(xq, sa, wq, sb)
    ref = x @ w.T
    N = w.shape[0]
    sx = np.repeat(sa.T.astype(np.float64), 128, axis=1)
    sw = np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    ex = np.abs(x) * 2.0 ** -4 * (1 + 2.0 ** -20) + sx * 2.0 ** -10
    ew = np.abs(w) * 2.0 ** -4 * (1 + 2.0 ** -20) + sw * 2.0 ** -10
    bound = ex @ np.abs(w).T + np.abs(x) @ ew.T + ex @ ew.T
    err = np.abs(y - ref)
    assert np.all(err <= bound * (1 + 1e-9) + 1e-12)
    # and the bound is not vacuous: typical error is far below |ref|
    assert np.median(err / (np.abs(x) @ np.abs(w).T)) < 0.02
    # a deliberately wrong activation-scale layout breaks the bound
    y_bad = oracle.gemm_nt(xq, np.ascontiguousarray(sa[::-1]), wq, sb)
    assert np.any(np.abs(y_bad - ref) > bound)


def test_kblock_permutation_invariance():
    rng = np.random.default_rng(26)
    M, N, K = 12, 130, 640
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = rng.uniform(0.1, 2, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.1, 2, (2, K // 128)).astype(np.float32)
    perm = np.array([3, 0, 4, 2, 1])
    kperm = (perm[:, None] * 128 + np.arange(128)).reshape(-1)
    y0 = oracle.gemm_nt(xq, sa, wq, sb)
    y1 = oracle.gemm_nt(np.ascontiguousarray(xq[:, kperm]), np.ascontiguousarray(sa[perm]),
                        np.ascontiguousarray(wq[:, kperm]), np.ascontiguousarray(sb[:, perm]))
    mag = oracle.gemm_nt(xq & 0x7F, sa, wq & 0x7F, sb)   # sum of |terms|
    assert np.all(np.abs(y0 - y1) <= 1e-14 * mag)


def test_elems_match_full():
    rng = np.random.default_rng(27)
    M, N, K = 33, 260, 256
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = rng.uniform(0.1, 2, (K // 128, M)).astype(np.float32)
    sb = rng.uniform(0.1, 2, (3, K // 128)).astype(np.float32)
    y = oracle.gemm_nt(xq, sa, wq, sb)
    mi = rng.integers(0, M, 100)
    ni = rng.integers(0, N, 100)
    assert np.array_equal(oracle.gemm_nt_elems(xq, sa, wq, sb, mi, ni), y[mi, ni])


def test_ue8m0_flag_reads_exponent_only():
    rng = np.random.default_rng(28)
    M, N, K = 8, 128, 256
    xq, wq = _codes(rng, (M, K)), _codes(rng, (N, K))
    sa = workloads.random_pow2(rng, (K // 128, M))
    sb = workloads.random_pow2(rng, (1, K // 128))
    y0 = oracle.gemm_nt(xq, sa, wq, sb)
    assert np.array_equal(oracle.gemm_nt(xq, sa, wq, sb, oracle.FLAG_UE8M0), y0)
    # a mantissa is ignored: 1.5 * 2^e reads as 2^e
    y1 = oracle.gemm_nt(xq, (sa * 1.5).astype(np.float32), wq, sb, oracle.FLAG_UE8M0)
    assert np.array_equal(y1, y0)


def test_exact_integer_case():
    """Small-integer inputs with power-of-two scales give exactly integer Y."""
    rng = np.random.default_rng(29)
    M, N, K = 8, 16, 256
    ints = np.array([0x00, 0x38, 0x40, 0x44, 0x48, 0xB8, 0xC0])   # 0, 1, 2, 3, 4, -1, -2
    xq = rng.choice(ints, (M, K)).astype(np.uint8)
    wq = rng.choice(ints, (N, K)).astype(np.uint8)
    sa = np.ones((2, M), np.float32)
    sb = np.ones((1, 2), np.float32)
    y = oracle.gemm_nt(xq, sa, wq, sb)
    assert np.array_equal(y, np.round(y))
    ia = DEC[xq].astype(np.int64)
    ib = DEC[wq].astype(np.int64)
    assert np.array_equal(y.astype(np.int64), ia @ ib.T)
