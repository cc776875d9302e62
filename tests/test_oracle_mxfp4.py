"""Pins of the MXFP4 weight oracle (E2M1 nibbles with one E8M0 scale per 1x32
group along K; tcgen05 page, sections 6.1 and 6.3; two 4-bit values packed
per byte along K, same page, section on operand majors).

The pages name the element format (E2M1: 1 sign, 2 exponent, 1 mantissa bit)
but print no values.  The decode table is pinned by a generic sign/exponent/
mantissa rule that must reproduce the page-pinned E4M3 table with 4 and 3
bits and then gives E2M1 with 2 and 1.  The GEMM is pinned to numpy's matmul
of the dequantised operands and to the already pinned MXFP8 GEMM."""
import numpy as np
import pytest

import oracle

DEC8 = oracle.e4m3_decode(np.arange(256))
DEC4 = oracle.e2m1_decode(np.arange(16))


def minifloat(code: int, ebits: int, mbits: int) -> float:
    """A sign/exponent/mantissa code with bias 2^(ebits-1) - 1 and gradual
    underflow, no infinities (the OCP-style narrow float formats)."""
    bias = (1 << (ebits - 1)) - 1
    s = (code >> (ebits + mbits)) & 1
    e = (code >> mbits) & ((1 << ebits) - 1)
    m = code & ((1 << mbits) - 1)
    mag = (m / (1 << mbits)) * 2.0 ** (1 - bias) if e == 0 else (1 + m / (1 << mbits)) * 2.0 ** (e - bias)
    return -mag if s else mag


def test_e2m1_decode_is_the_minifloat_rule_that_gives_e4m3():
    finite8 = [c for c in range(256) if (c & 0x7F) != 0x7F]
    assert all(minifloat(c, 4, 3) == DEC8[c] for c in finite8)     # the rule, checked on E4M3
    assert [minifloat(c, 2, 1) for c in range(16)] == list(DEC4)   # ... gives the E2M1 table
    assert DEC4[7] == 6.0 and DEC4[1] == 0.5


def test_e2m1_encode_round_trip_ties_and_saturation():
    for c in range(16):
        assert oracle.e2m1_encode(np.float32(DEC4[c])) == c        # -0 keeps its sign (8)
    mags = DEC4[:8]
    for c in range(7):                                              # every midpoint to the even code
        mid = np.float32((mags[c] + mags[c + 1]) / 2)
        assert oracle.e2m1_encode(mid) == (c if c % 2 == 0 else c + 1)
        assert oracle.e2m1_encode(-mid) == 8 | (c if c % 2 == 0 else c + 1)
    assert oracle.e2m1_encode(np.float32(6.5)) == 7 and oracle.e2m1_encode(np.float32(1e9)) == 7
    grid = np.linspace(0, 7, 2001).astype(np.float32)
    codes = oracle.e2m1_encode(grid)
    assert np.all(np.diff(DEC4[codes]) >= 0)                        # monotone
    assert np.all(np.abs(DEC4[codes] - np.minimum(grid, 6)) <= 0.5 * np.where(grid < 2, 0.5, np.where(grid < 4, 1, 2)) + 1e-7)


def unpack(q):
    return np.stack([q & 0xF, q >> 4], axis=-1).reshape(q.shape[0], -1)


def test_mxfp4_quantizer_properties():
    rng = np.random.default_rng(8)
    R, K = 40, 1024
    x = (rng.standard_normal((R, K)) * np.exp2(rng.integers(-10, 10, (R, 1)))).astype(np.float32)
    x[rng.random((R, K)) < 0.002] *= 100
    x[5, 32:64] = 0.0
    q, e = oracle.quant_mxfp4(x)
    assert q.shape == (R, K // 2) and e.shape == (R, K // 32)
    nib = unpack(q)
    s = np.repeat(np.ldexp(1.0, e.astype(np.int64) - 127), 32, axis=1)
    amax = np.abs(x).reshape(R, K // 32, 32).max(axis=2)
    t = np.maximum(amax, np.float32(1e-4)).astype(np.float32) / np.float32(6.0)
    sg = np.ldexp(1.0, e.astype(np.int64) - 127)
    assert np.all(sg >= t) and np.all(sg / 2 < t)                   # least power of two >= amax/6
    v = x / s                                                        # exact: s is a power of two
    d = DEC4[nib]
    step = np.where(np.abs(v) < 2, 0.5, np.where(np.abs(v) < 4, 1.0, 2.0))
    assert np.all(np.abs(d - v) <= step / 2 + 1e-6)                 # nearest E2M1 value
    gmax = np.abs(d).reshape(R, K // 32, 32).max(axis=2)
    live = amax >= 1e-4
    assert np.all((gmax[live] >= 3) & (gmax[live] <= 6))
    assert np.all(nib[5, 32:64] == 0)
    x2 = x.copy()
    x2[7, 300] *= 40
    q2, e2 = oracle.quant_mxfp4(x2)
    de = np.argwhere(e != e2)
    assert len(de) == 1 and tuple(de[0]) == (7, 300 // 32)
    dq = np.argwhere(unpack(q) != unpack(q2))
    assert np.all(dq[:, 0] == 7) and np.all(dq[:, 1] // 32 == 300 // 32)


@pytest.mark.parametrize("M,N,K", [(5, 7, 96), (3, 11, 256), (16, 4, 32)])
def test_gemm_mx_w4_equals_dequantised_matmul(M, N, K):
    rng = np.random.default_rng(M * 31 + N)
    finite = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    xq = rng.choice(finite, (M, K)).astype(np.uint8)
    wq = rng.integers(0, 256, (N, K // 2)).astype(np.uint8)
    ea = rng.integers(110, 140, (M, K // 32)).astype(np.uint8)
    eb = rng.integers(110, 140, (N, K // 32)).astype(np.uint8)
    xd = DEC8[xq] * np.repeat(np.ldexp(1.0, ea.astype(np.int64) - 127), 32, axis=1)
    wd = DEC4[unpack(wq)] * np.repeat(np.ldexp(1.0, eb.astype(np.int64) - 127), 32, axis=1)
    ref = np.matmul(xd, wd.T)
    y = oracle.gemm_mx_w4(xq, ea, wq, eb)
    assert np.all(np.abs(y - ref) <= 1e-12 * (np.abs(xd) @ np.abs(wd).T) + 1e-300)
    mi, ni = rng.integers(0, M, 40), rng.integers(0, N, 40)
    assert np.array_equal(oracle.gemm_mx_w4_elems(xq, ea, wq, eb, mi, ni), y[mi, ni])


def test_gemm_mx_w4_equals_the_mxfp8_gemm_with_w_as_e4m3():
    """Every E2M1 value is an E4M3 value: re-encoding W's elements as E4M3
    gives the same products, so the pinned MXFP8 GEMM must agree exactly."""
    rng = np.random.default_rng(12)
    x = rng.standard_normal((24, 512)).astype(np.float32)
    w = rng.standard_normal((40, 512)).astype(np.float32)
    xq, ea = oracle.quant_mx(x)
    wq4, eb = oracle.quant_mxfp4(w)
    w8 = oracle.e4m3_encode(DEC4[unpack(wq4)].astype(np.float32))
    assert np.array_equal(DEC8[w8], DEC4[unpack(wq4)])
    assert np.array_equal(oracle.gemm_mx_w4(xq, ea, wq4, eb), oracle.gemm_mx(xq, ea, w8, eb))
