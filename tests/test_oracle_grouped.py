"""Pins for the oracle's grouped (MoE) GEMMs (CPU only).

Grouped outputs must equal per-expert dense GEMMs on the sliced inputs, and
rows outside the valid set must not be written.
"""
import numpy as np

import oracle
import workloads


def _quant_all(wl):
    xq, sa = oracle.quant_1x128(wl.x, oracle.FLAG_UE8M0 if wl.ue8m0 else 0)
    wq, sb = oracle.quant_128x128(wl.w, oracle.FLAG_UE8M0 if wl.ue8m0 else 0)
    return xq, sa, wq, sb


def test_contiguous_equals_per_expert_dense():
    wl = workloads.contiguous(E=4, tokens=300, N=256, K=256, seed=31,
                              counts=np.array([0, 130, 1, 169]))
    assert wl.M == 0 + 256 + 128 + 256
    assert oracle.contiguous_layout_violations(wl.m_indices, wl.E) == 0
    xq, sa, wq, sb = _quant_all(wl)
    y, written = oracle.grouped_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E)
    assert np.array_equal(written, wl.m_indices >= 0)
    N, K = wl.N, wl.K
    KB, NB = K // 128, N // 128
    for e in range(wl.E):
        rows = np.nonzero(wl.m_indices == e)[0]
        if len(rows) == 0:
            continue
        ref = oracle.gemm_nt(xq[rows], np.ascontiguousarray(sa[:, rows]),
                             wq[e * N:(e + 1) * N], sb[e * NB:(e + 1) * NB])
        assert np.array_equal(y[rows], ref)
    assert np.all(y[~written] == 0)


def test_contiguous_foreign_and_out_of_range_rows_skipped():
    M, N, K, E = 256, 128, 128, 3
    rng = np.random.default_rng(32)
    xq = workloads.random_codes(rng, (M, K))
    wq = workloads.random_codes(rng, (E * N, K))
    sa = np.ones((1, M), np.float32)
    sb = np.ones((E, 1), np.float32)
    idx = np.full(M, -1, np.int32)
    idx[0:5] = 7          # out of range: skipped
    idx[5:100] = 1        # block expert of rows 0..127 is 1 (first valid index)
    idx[100:110] = 2      # foreign rows inside expert 1's block: skipped
    idx[128:256] = 0
    assert oracle.contiguous_layout_violations(idx, E) == 1
    y, written = oracle.grouped_contiguous(xq, sa, wq, sb, idx, E)
    expect = np.zeros(M, bool)
    expect[5:100] = True
    expect[128:256] = True
    assert np.array_equal(written, expect)
    ref1 = oracle.gemm_nt(xq[5:100], np.ascontiguousarray(sa[:, 5:100]), wq[N:2 * N], sb[1:2])
    assert np.array_equal(y[5:100], ref1)


def test_masked_equals_per_expert_dense_and_clamps():
    E, max_m, N, K = 5, 40, 256, 384
    mm = np.array([0, 40, 17, -3, 99], np.int32)      # -3 -> 0, 99 -> 40
    wl = workloads.masked(E, max_m, N, K, seed=33, ue8m0=True, masked_m=mm)
    xq, sa, wq, sb = _quant_all(wl)
    y, written = oracle.grouped_masked(xq, sa, wq, sb, mm, E, max_m, oracle.FLAG_UE8M0)
    valid = np.clip(mm, 0, max_m)
    expect = np.concatenate([np.arange(max_m) < v for v in valid])
    assert np.array_equal(written, expect)
    NB = N // 128
    for e in range(E):
        if valid[e] == 0:
            continue
        rows = np.arange(e * max_m, e * max_m + valid[e])
        ref = oracle.gemm_nt(xq[rows], np.ascontiguousarray(sa[:, rows]),
                             wq[e * N:(e + 1) * N], sb[e * NB:(e + 1) * NB], oracle.FLAG_UE8M0)
        assert np.array_equal(y[rows], ref)
    assert np.all(y[~written] == 0)


def test_alignment_fact():
    """DeepGEMM page, grouped-layout section: each expert segment of the
    contiguous layout is aligned to the GEMM's M block; the generator pads
    every segment to 128 rows."""
    wl = workloads.contiguous(E=8, tokens=1000, N=128, K=128, seed=34)
    starts = [np.nonzero(wl.m_indices == e)[0] for e in range(8)]
    for s in starts:
        if len(s):
            assert s[0] % 128 == 0
    assert wl.M % 128 == 0
    assert int((wl.m_indices >= 0).sum()) == 1000
