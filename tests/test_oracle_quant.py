"""Pins for the oracle's 1x128 / 128x128 quantizers (CPU only).

Pinned against the DeepGEMM page's worked outlier example
(tests/golden/deepgemm_outlier_example.json) and against properties that any
correct absmax/448 block quantizer has: codes within +-448, every nonzero
group reaching 448, confinement of an outlier to its own group, and an
element-wise dequantization error within half an E4M3 step.
"""
import json
import os

import numpy as np
import pytest

import oracle
import workloads

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
DEC = oracle.e4m3_decode(np.arange(256))


def _dequant_1x128(xq, sa):
    M, K = xq.shape
    return DEC[xq] * np.repeat(sa.T.astype(np.float64), 128, axis=1)


def _dequant_128x128(wq, sb):
    N, K = wq.shape
    s = np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    return DEC[wq] * s


def test_worked_outlier_example():
    g = json.load(open(os.path.join(GOLDEN, "deepgemm_outlier_example.json")))
    p = g["printed"]
    rng = np.random.default_rng(7)
    x = rng.uniform(-p["others_abs_max"], p["others_abs_max"], (1, p["block_size"]))
    x = x.astype(np.float32)
    x[0, 5] = p["outlier"]
    x[0, 9] = p["others_abs_max"]
    xq, sa = oracle.quant_1x128(x)
    s = float(sa[0, 0])
    assert abs(s - p["scale_approx"]) < g["tolerances"]["scale_approx_abs"]
    assert np.float32(s) == np.float32(p["outlier"]) / np.float32(p["e4m3_max"])
    ratio = p["others_abs_max"] / s
    assert abs(ratio - p["ratio_approx"]) < g["tolerances"]["ratio_approx_abs"]
    assert xq[0, 5] == 0x7E
    assert xq[0, 9] == 0x39 and DEC[0x39] == 1.125
    # every "normal" entry lands in the bottom of the E4M3 range (|q| <= 1.125)
    others = np.delete(xq[0], 5)
    assert np.all(np.abs(DEC[others]) <= 1.125)


@pytest.mark.parametrize("flags", [0, oracle.FLAG_UE8M0])
def test_1x128_invariants(flags):
    wl = workloads.dense(96, 8, 640, seed=11, outlier_frac=0.01, outlier_mult=50.0)
    x = wl.x
    xq, sa = oracle.quant_1x128(x, flags)
    M, K = x.shape
    assert sa.shape == (K // 128, M)
    vals = DEC[xq]
    assert np.all(np.isfinite(vals)) and np.all(np.abs(vals) <= 448)
    g = x.reshape(M, K // 128, 128)
    amax = np.abs(g).max(axis=2).T                          # (KB, M)
    qmax = np.abs(vals.reshape(M, K // 128, 128)).max(axis=2).T
    s_plain = np.maximum(amax, np.float32(1e-4)) / np.float32(448)
    if flags == 0:
        assert np.array_equal(sa, s_plain.astype(np.float32))
        assert np.all(qmax == 448)
    else:
        m, e = np.frexp(sa)
        assert np.all(m == 0.5), "UE8M0 scales must be powers of two"
        assert np.all(sa >= s_plain) and np.all(sa < 2 * s_plain)
        # amax/s lies in (224, 448]; E4M3 rounding can bring it down to 224
        assert np.all((qmax >= 224) & (qmax <= 448))
    # element-wise error: half an E4M3 step (relative 2^-4) or half the
    # subnormal step s*2^-10, plus the binary32 rounding of x/s
    err = np.abs(_dequant_1x128(xq, sa) - x.astype(np.float64))
    s_el = np.repeat(sa.T.astype(np.float64), 128, axis=1)
    bound = np.abs(x) * 2.0 ** -4 * (1 + 2.0 ** -20) + s_el * 2.0 ** -10
    assert np.all(err <= bound)


@pytest.mark.parametrize("flags", [0, oracle.FLAG_UE8M0])
def test_128x128_invariants_ragged_n(flags):
    wl = workloads.dense(4, 300, 384, seed=12, outlier_frac=0.01, outlier_mult=50.0)
    w = wl.w
    wq, sb = oracle.quant_128x128(w, flags)
    N, K = w.shape
    assert sb.shape == (3, 3)
    vals = DEC[wq]
    assert np.all(np.abs(vals) <= 448)
    for nb in range(3):
        for kb in range(3):
            blk = w[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            qb = vals[nb * 128:(nb + 1) * 128, kb * 128:(kb + 1) * 128]
            s_plain = np.float32(max(np.abs(blk).max(), np.float32(1e-4))) / np.float32(448)
            if flags == 0:
                assert sb[nb, kb] == s_plain
                assert np.abs(qb).max() == 448
            else:
                assert np.frexp(sb[nb, kb])[0] == 0.5
                assert s_plain <= sb[nb, kb] < 2 * s_plain
    err = np.abs(_dequant_128x128(wq, sb) - w.astype(np.float64))
    s_el = np.repeat(np.repeat(sb.astype(np.float64), 128, axis=0)[:N], 128, axis=1)
    assert np.all(err <= np.abs(w) * 2.0 ** -4 * (1 + 2.0 ** -20) + s_el * 2.0 ** -10)


def test_outlier_confined_to_its_group():
    """DeepGEMM page, outlier section: each group has its own scale, so an
    outlier cannot disturb any other group."""
    wl = workloads.dense(8, 256, 512, seed=13)
    x, w = wl.x.copy(), wl.w.copy()
    xq0, sa0 = oracle.quant_1x128(x)
    wq0, sb0 = oracle.quant_128x128(w)
    x[3, 200] *= 50
    w[130, 300] *= 50
    xq1, sa1 = oracle.quant_1x128(x)
    wq1, sb1 = oracle.quant_128x128(w)
    dx = np.argwhere(xq0 != xq1)
    assert len(dx) > 0 and np.all(dx[:, 0] == 3) and np.all(dx[:, 1] // 128 == 1)
    assert np.argwhere(sa0 != sa1).tolist() == [[1, 3]]
    dw = np.argwhere(wq0 != wq1)
    assert len(dw) > 0 and np.all(dw[:, 0] // 128 == 1) and np.all(dw[:, 1] // 128 == 2)
    assert np.argwhere(sb0 != sb1).tolist() == [[1, 2]]


def test_zero_group_floor_and_signs():
    x = np.zeros((2, 256), np.float32)
    x[1, :128] = -0.0
    x[1, 128:] = -1.0
    xq, sa = oracle.quant_1x128(x)
    assert np.all(sa[0] == np.float32(1e-4) / np.float32(448))
    assert np.all(xq[0] == 0) and np.all(xq[1, :128] == 0x80)
    assert np.all(xq[1, 128:] == 0xFE) and sa[1, 1] == np.float32(1) / np.float32(448)


def test_bad_shape_rejected():
    with pytest.raises(ValueError):
        oracle.quant_1x128(np.zeros((2, 100), np.float32))
