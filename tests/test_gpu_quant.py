"""GPU quantizers against the oracle: codes and scale bits must be identical."""
import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import dev, host, say

pytestmark = pytest.mark.gpu


def _q1(x, flags):
    say(f"quant_1x128 M={x.shape[0]} K={x.shape[1]} flags={flags}")
    xq, sa = fp8.quant_1x128(dev(x), ue8m0=bool(flags))
    return host(xq), host(sa)


def _q2(w, flags):
    say(f"quant_128x128 N={w.shape[0]} K={w.shape[1]} flags={flags}")
    wq, sb = fp8.quant_128x128(dev(w), ue8m0=bool(flags))
    return host(wq), host(sb)


@pytest.mark.parametrize("M,K,flags", [(128, 512, 0), (1, 128, 0), (300, 1024, 0),
                                       (77, 384, 1), (128, 512, 1), (9, 7168, 0),
                                       # a row of 8-group units plus a short one
                                       (33, 1280, 0), (5, 1664, 1)])
def test_quant_1x128_bitexact(M, K, flags):
    wl = workloads.dense(M, 1, K, seed=100 + M, outlier_frac=0.01, outlier_mult=50.0)
    xq_ref, sa_ref = oracle.quant_1x128(wl.x, flags)
    xq, sa = _q1(wl.x, flags)
    assert np.array_equal(xq, xq_ref)
    assert np.array_equal(sa.view(np.uint32), sa_ref.view(np.uint32))


@pytest.mark.parametrize("N,K,flags", [(256, 512, 0), (300, 384, 0), (1, 128, 0),
                                       (129, 256, 1), (512, 1024, 1)])
def test_quant_128x128_bitexact(N, K, flags):
    wl = workloads.dense(1, N, K, seed=200 + N, outlier_frac=0.01, outlier_mult=50.0)
    wq_ref, sb_ref = oracle.quant_128x128(wl.w, flags)
    wq, sb = _q2(wl.w, flags)
    assert np.array_equal(wq, wq_ref)
    assert np.array_equal(sb.view(np.uint32), sb_ref.view(np.uint32))


def _encoder_cases() -> np.ndarray:
    """FP32 values that stress the E4M3 encoder: every code's value, every
    midpoint and its fp32 neighbours, random values over the whole range,
    tiny values, signed zeros."""
    dec = oracle.e4m3_decode(np.arange(0x7F))
    mid = ((dec[:-1] + dec[1:]) / 2).astype(np.float32)
    vals = [dec.astype(np.float32), mid]
    for k in (1, 2, 3):
        up, dn = mid.copy(), mid.copy()
        for _ in range(k):
            up = np.nextafter(up, np.float32(np.inf))
            dn = np.nextafter(dn, np.float32(0))
        vals += [up, dn]
    rng = np.random.default_rng(5)
    vals.append(rng.uniform(0, 448, 60000).astype(np.float32))
    vals.append(np.exp2(rng.uniform(-30, 9, 60000)).astype(np.float32))
    vals.append(np.array([0.0, 1e-45, 1e-38, 2.0 ** -10, 447.9999, 448.0], np.float32))
    v = np.concatenate(vals)
    v = v[np.abs(v) <= 448]
    return np.concatenate([v, -v])


def test_hardware_encoder_matches_oracle():
    """Each 128-group carries 448 in its first slot, so its scale is exactly 1
    and the other 127 slots are encoded as given."""
    v = _encoder_cases()
    per = 127
    G = (v.size + per - 1) // per
    v = np.concatenate([v, np.zeros(G * per - v.size, np.float32)])
    x = np.empty((G, 128), np.float32)
    x[:, 0] = 448.0
    x[:, 1:] = v.reshape(G, per)
    xq_ref, sa_ref = oracle.quant_1x128(x)
    assert np.all(sa_ref == 1.0)
    xq, sa = _q1(x, 0)
    assert np.all(sa == 1.0)
    bad = np.argwhere(xq != xq_ref)
    assert len(bad) == 0, [(x[tuple(b)], xq[tuple(b)], xq_ref[tuple(b)]) for b in bad[:8]]


def _near_boundaries(c):
    """(values, group maximum) for a scale factor c in [1, 2): the group's
    maximum is c*448, so its scale s = fl32(max/448) is not a power of two,
    and the values put the quotient x / s on every E4M3 rounding boundary
    (the midpoint between two neighbouring codes) below 440 and within 10
    FP32 units either side of it, both signs."""
    amax = np.float32(448 * c)
    s = np.float32(amax / np.float32(448))
    dec = oracle.e4m3_decode(np.arange(0x7F)).astype(np.float64)
    mid = (dec[:-1] + dec[1:]) / 2
    base = (mid[mid < 440] * np.float64(s)).astype(np.float32).view(np.int32)
    v = np.concatenate([(base + k).view(np.float32) for k in range(-10, 11)])
    return np.concatenate([v, -v]), amax, s


def test_quotients_on_rounding_boundaries():
    """Codes where x / s lies on or next to an E4M3 rounding boundary, with
    scales that are not powers of two: the quantizers take the product with
    the reciprocal only where it provably rounds like the correctly rounded
    quotient, and divide elsewhere; both must match the oracle's division
    bit for bit."""
    rng = np.random.default_rng(9)
    rows, blocks = [], []
    for c in rng.uniform(1.0, 2.0, 8):
        v, amax, s = _near_boundaries(c)
        rng.shuffle(v)
        per = 127
        n = (v.size + per - 1) // per
        r = np.empty((n, 128), np.float32)
        r[:, 0] = amax
        r[:, 1:] = np.resize(v, n * per).reshape(n, per)
        rows.append(r)
        b = np.resize(v, 128 * 128).reshape(128, 128).astype(np.float32)
        b[0, 0] = amax
        blocks.append(b)
    x = np.concatenate(rows)
    xq_ref, sa_ref = oracle.quant_1x128(x)
    xq, sa = _q1(x, 0)
    assert np.array_equal(sa.view(np.uint32), sa_ref.view(np.uint32))
    bad = np.argwhere(xq != xq_ref)
    assert len(bad) == 0, [(x[tuple(b)], xq[tuple(b)], xq_ref[tuple(b)]) for b in bad[:8]]
    w = np.concatenate(blocks)                     # (8*128, 128): one block per factor
    wq_ref, sb_ref = oracle.quant_128x128(w)
    assert len(np.unique(sb_ref)) == len(blocks)
    wq, sb = _q2(w, 0)
    assert np.array_equal(sb.view(np.uint32), sb_ref.view(np.uint32))
    bad = np.argwhere(wq != wq_ref)
    assert len(bad) == 0, [(w[tuple(b)], wq[tuple(b)], wq_ref[tuple(b)]) for b in bad[:8]]


def test_zero_and_negative_zero_groups():
    x = np.zeros((4, 256), np.float32)
    x[1] = -0.0
    x[2, :128] = -1e-30
    x[3, 5] = 3.0
    for flags in (0, 1):
        xq_ref, sa_ref = oracle.quant_1x128(x, flags)
        xq, sa = _q1(x, flags)
        assert np.array_equal(xq, xq_ref)
        assert np.array_equal(sa.view(np.uint32), sa_ref.view(np.uint32))


@pytest.mark.slow
@pytest.mark.parametrize("cfg", [1, 2, 3, 4, 5])
def test_quantizers_full_size_configs(cfg):
    wl = workloads.config(cfg)
    flags = 1 if wl.ue8m0 else 0
    say(f"config {cfg}: oracle quantization ({wl.x.size + wl.w.size} elements)")
    xq_ref, sa_ref = oracle.quant_1x128(wl.x, flags)
    xq, sa = _q1(wl.x, flags)
    assert np.array_equal(xq, xq_ref)
    assert np.array_equal(sa.view(np.uint32), sa_ref.view(np.uint32))
    del xq, sa, xq_ref, sa_ref
    wq_ref, sb_ref = oracle.quant_128x128(wl.w, flags)
    wq, sb = _q2(wl.w, flags)
    assert np.array_equal(wq, wq_ref)
    assert np.array_equal(sb.view(np.uint32), sb_ref.view(np.uint32))
