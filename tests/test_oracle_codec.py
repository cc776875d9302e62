"""Pins for the oracle's E4M3 codec (CPU only).

Pinned against: the page's printed format facts (tests/golden/e4m3_format.json),
the closed form over all 256 codes, torch's float8_e4m3fn conversion (an
independent library routine), and properties any correct nearest-even encoder
must have (round trip, monotonicity, midpoints to the even code).
"""
import json
import os

import numpy as np
import pytest
import torch

import oracle

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")


def _torch_decode_all():
    codes = torch.arange(256, dtype=torch.int32).to(torch.uint8)
    return codes.view(torch.float8_e4m3fn).to(torch.float64).numpy()


def _torch_encode(v):
    t = torch.from_numpy(np.ascontiguousarray(v, dtype=np.float32))
    return t.to(torch.float8_e4m3fn).view(torch.uint8).numpy()


def test_page_format_facts():
    g = json.load(open(os.path.join(GOLDEN, "e4m3_format.json")))
    dec = oracle.e4m3_decode(np.arange(256))
    finite = dec[np.isfinite(dec)]
    assert finite.max() == g["facts"]["max_finite"]
    assert finite[finite > 0].min() == g["facts"]["min_subnormal"]
    assert oracle.e4m3_decode(0x7E) == g["derived_codes"]["0x7e"]
    assert oracle.e4m3_decode(0x01) == g["derived_codes"]["0x01"]
    # 2^(exponent_bits + mantissa_bits + 1) patterns, two of them NaN (S.1111.111)
    assert np.isnan(dec).sum() == 2
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])


def test_decode_matches_torch_all_codes():
    ours = oracle.e4m3_decode(np.arange(256))
    ref = _torch_decode_all()
    both_nan = np.isnan(ours) & np.isnan(ref)
    assert np.array_equal(ours[~both_nan], ref[~both_nan])
    assert np.array_equal(np.signbit(ours[~both_nan]), np.signbit(ref[~both_nan]))


def test_decode_closed_form_sign_symmetry_and_order():
    dec = oracle.e4m3_decode(np.arange(256))
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0), "positive codes must increase strictly"
    assert np.array_equal(dec[0x80:0xFF], -pos)
    # subnormals are evenly spaced by 2^-9, normals have 8 steps per binade
    assert np.array_equal(pos[:8], np.arange(8) * 2.0 ** -9)
    for e in range(1, 16):
        lo = pos[8 * e]
        assert lo == 2.0 ** (e - 7)


def test_encode_round_trip_every_finite_code():
    codes = np.array([c for c in range(256) if (c & 0x7F) != 0x7F], np.uint8)
    vals = oracle.e4m3_decode(codes).astype(np.float32)
    assert np.array_equal(oracle.e4m3_encode(vals), codes)


def test_encode_midpoints_go_to_even_code():
    dec = oracle.e4m3_decode(np.arange(0x7F))
    mid = (dec[:-1] + dec[1:]) / 2           # exact in fp32 (one extra bit)
    mid32 = mid.astype(np.float32)
    assert np.array_equal(mid32.astype(np.float64), mid)
    got = oracle.e4m3_encode(mid32)
    lo = np.arange(0x7E)
    expect = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, expect)
    # one fp32 ulp either side of the midpoint leaves the tie
    below = np.nextafter(mid32, np.float32(0))
    above = np.nextafter(mid32, np.float32(np.inf))
    assert np.array_equal(oracle.e4m3_encode(below[1:]), lo[1:])
    assert np.array_equal(oracle.e4m3_encode(above), lo + 1)


def test_encode_matches_torch_in_range():
    rng = np.random.default_rng(0)
    v = np.concatenate([
        rng.uniform(-448, 448, 200000),
        rng.standard_normal(200000) * np.exp2(rng.uniform(-14, 9, 200000)),
        np.exp2(rng.uniform(-20, -8, 20000)) * rng.choice([-1, 1], 20000),
    ]).astype(np.float32)
    v = v[np.abs(v) <= 448]
    assert np.array_equal(oracle.e4m3_encode(v), _torch_encode(v))


def test_encode_saturates_and_keeps_sign():
    big = np.array([448, 448.5, 463.9, 464, 465, 480, 1e4, 3e38], np.float32)
    assert np.all(oracle.e4m3_encode(big) == 0x7E)
    assert np.all(oracle.e4m3_encode(-big) == 0xFE)
    tiny = np.array([0.0, 1e-30, 2.0 ** -11], np.float32)
    assert np.all(oracle.e4m3_encode(tiny) == 0x00)
    assert np.all(oracle.e4m3_encode(-tiny) == 0x80)
    # 2^-10 is the midpoint between 0 and 2^-9: ties to the even code 0
    assert oracle.e4m3_encode(np.float32(2.0 ** -10)) == 0x00
    assert oracle.e4m3_encode(np.float32(2.0 ** -10 * 1.0001)) == 0x01


def test_encode_monotone():
    rng = np.random.default_rng(1)
    v = np.sort(rng.uniform(-460, 460, 100000).astype(np.float32))
    d = oracle.e4m3_decode(oracle.e4m3_encode(v))
    assert np.all(np.diff(d) >= 0)


def test_products_exact_in_fp32():
    """DeepGEMM page, section on the two GEMM-level problems: the product of two
    E4M3 values needs at most 8 significant bits and is exact in FP32."""
    dec = oracle.e4m3_decode(np.arange(256))
    ok = np.isfinite(dec)
    a = dec[ok]
    p64 = np.multiply.outer(a, a)
    p32 = np.multiply.outer(a.astype(np.float32), a.astype(np.float32))
    assert np.array_equal(p32.astype(np.float64), p64)
