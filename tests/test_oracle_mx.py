"""Pins of the MXFP8 oracle (E4M3 elements, one E8M0 scale per 1x32 group
along K on both operands; tcgen05 page, sections 6.1 and 6.3).

Each test checks the oracle against something other than itself: the already
pinned 1x128 UE8M0 quantizer in the special case where the two coincide,
properties fixed by the definition of the scale, and the dequantise-then-
multiply form of the GEMM computed by numpy's matmul."""
import numpy as np
import pytest

import oracle

DEC = oracle.e4m3_decode(np.arange(256))


def test_mx_reduces_to_1x128_ue8m0_when_every_subgroup_holds_the_group_max():
    # Every 32-subgroup of every 128-group holds an entry of the group's
    # largest magnitude: the MX scales then equal the 1x128 UE8M0 scale and
    # the codes are the same bytes.
    rng = np.random.default_rng(1)
    M, K = 9, 640
    x = rng.standard_normal((M, K)).astype(np.float32)
    x[rng.random((M, K)) < 0.02] *= 50
    for m in range(M):
        for kb in range(K // 128):
            g = x[m, kb * 128:(kb + 1) * 128]
            amax = np.abs(g).max()
            for j in range(4):
                pos = 32 * j + (7 * j + m) % 32
                g[pos] = amax if g[pos] >= 0 else -amax
    q_mx, e_mx = oracle.quant_mx(x)
    q_1, sa = oracle.quant_1x128(x, oracle.FLAG_UE8M0)
    assert np.array_equal(q_mx, q_1)
    s_mx = np.ldexp(1.0, e_mx.astype(np.int64) - 127).astype(np.float32)   # (M, K/32)
    s_1 = np.repeat(sa.T, 4, axis=1)                                       # (M, K/32)
    assert np.array_equal(s_mx.view(np.uint32), s_1.view(np.uint32))


def test_mx_scale_is_the_least_power_of_two_at_or_above_amax_over_448():
    rng = np.random.default_rng(2)
    R, K = 33, 2048
    x = (rng.standard_normal((R, K)) * np.exp2(rng.integers(-12, 12, (R, 1)))).astype(np.float32)
    x[rng.random((R, K)) < 0.001] *= 100
    x[3, 64:96] = 0.0                      # an all-zero group: amax floored at 1e-4
    x[4, 0:32] = np.float32(1e-6)          # a tiny group, also floored
    q, e = oracle.quant_mx(x)
    amax = np.abs(x).reshape(R, K // 32, 32).max(axis=2)
    a = np.maximum(amax, np.float32(1e-4)).astype(np.float32)
    t = a / np.float32(448.0)                                   # binary32 quotient
    s = np.ldexp(1.0, e.astype(np.int64) - 127)
    assert np.all(s >= t) and np.all(s / 2 < t)
    mag = np.abs(DEC[q]).reshape(R, K // 32, 32).max(axis=2)
    assert np.all((q & 0x7F) <= 0x7E)                           # no NaN code, |q| <= 448
    live = amax >= 1e-4
    # amax/s lies in (224, 448]; E4M3 rounding can bring it down to 224
    assert np.all(mag[live] >= 224) and np.all(mag[live] <= 448)
    assert np.all(q[3, 64:96] == 0) and e[3, 2] == e[4, 0]


def test_mx_outlier_changes_only_its_own_group():
    rng = np.random.default_rng(3)
    x = rng.standard_normal((4, 512)).astype(np.float32)
    q0, e0 = oracle.quant_mx(x)
    x2 = x.copy()
    x2[2, 200] *= 50
    q1, e1 = oracle.quant_mx(x2)
    dq = np.argwhere(q0 != q1)
    de = np.argwhere(e0 != e1)
    assert len(de) == 1 and tuple(de[0]) == (2, 200 // 32)
    assert len(dq) > 0 and np.all(dq[:, 0] == 2) and np.all(dq[:, 1] // 32 == 200 // 32)


@pytest.mark.parametrize("M,N,K", [(5, 7, 96), (3, 11, 256), (17, 4, 32)])
def test_mx_gemm_equals_dequantised_matmul(M, N, K):
    rng = np.random.default_rng(M * 100 + N)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    xq = rng.choice(finite, (M, K)).astype(np.uint8)
    wq = rng.choice(finite, (N, K)).astype(np.uint8)
    ea = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    eb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    xd = DEC[xq] * np.repeat(np.ldexp(1.0, ea.astype(np.int64) - 127), 32, axis=1)
    wd = DEC[wq] * np.repeat(np.ldexp(1.0, eb.astype(np.int64) - 127), 32, axis=1)
    ref = np.matmul(xd, wd.T)
    y = oracle.gemm_mx(xq, ea, wq, eb)
    tol = 1e-12 * (np.abs(xd) @ np.abs(wd).T) + 1e-300
    assert np.all(np.abs(y - ref) <= tol)
    mi, ni = rng.integers(0, M, 50), rng.integers(0, N, 50)
    assert np.array_equal(oracle.gemm_mx_elems(xq, ea, wq, eb, mi, ni), y[mi, ni])


def test_mx_gemm_of_quantised_data_approximates_the_fp32_product():
    # End to end: E4M3 with a per-32 power-of-two scale carries 3 mantissa
    # bits, so each product is within about 2 * 2^-4 relative of the FP32 one.
    rng = np.random.default_rng(4)
    x = rng.standard_normal((16, 512)).astype(np.float32)
    w = rng.standard_normal((24, 512)).astype(np.float32)
    xq, ea = oracle.quant_mx(x)
    wq, eb = oracle.quant_mx(w)
    y = oracle.gemm_mx(xq, ea, wq, eb)
    ref = x.astype(np.float64) @ w.astype(np.float64).T
    bound = 0.13 * (np.abs(x).astype(np.float64) @ np.abs(w).astype(np.float64).T)
    assert np.all(np.abs(y - ref) <= bound)


def test_mx_rejects_k_not_a_multiple_of_32():
    with pytest.raises(ValueError):
        oracle.quant_mx(np.zeros((2, 48), np.float32))
