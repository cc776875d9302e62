"""Host-side replay of the contiguous layout's pair schedule (no GPU).

Every workgroup of the three contiguous launches builds the same schedule from
the row indices on the device (gemm_common.h: build_pair_sched, pair_share).
This replays that rule in Python and checks it over random block layouts and
over the MoE workload's own layout:
  * every 128-row block that names an expert is computed exactly once, by one
    of the three launches, and a block of padding rows only by none;
  * a pair is two consecutive blocks of one expert, paired in order within
    their run;
  * the first two launches hold whole rounds of tiles whenever they pass work
    on, and keep everything otherwise.
The launches' results are checked against the oracle on the GPU
(test_gpu_grouped.py); this pins the rule they share and the split the
design notes quote for the 8-expert workload.
"""
import numpy as np
import pytest

import fine_grained_block_e4m3_amd as fp8
import workloads

CUS = 256


def block_experts(idx, E):
    """Expert of each 128-row block: the first index in [0, E) among its rows."""
    out = []
    for r0 in range(0, len(idx), 128):
        v = [int(x) for x in idx[r0:r0 + 128] if 0 <= x < E]
        out.append(v[0] if v else -1)
    return out


def pairs_and_singles(be):
    pairs, singles = [], []
    run_start, prev = 0, -1
    for b, e in enumerate(be):
        if e >= 0 and e != prev:
            run_start = b
        prev = e
        if e < 0 or (b - run_start) % 2:
            continue
        nxt = be[b + 1] if b + 1 < len(be) else -1
        (pairs if nxt == e else singles).append(b)
    return pairs, singles


def units_kept(units, nt, cus):
    tiles = units * nt
    full, last = divmod(tiles, cus)
    return full * cus // nt if 2 * last < cus else units


def shares(be, N, cus=CUS):
    """Blocks of each launch: (256-row pairs, 128x256 blocks, 128x64 blocks)."""
    pairs, singles = pairs_and_singles(be)
    nt = (N + 255) // 256
    pm = units_kept(len(pairs), nt, cus)
    left = singles + [b + j for b in pairs[pm:] for j in (0, 1)]
    mid = units_kept(len(left), nt, cus)
    return pairs[:pm], left[:mid], left[mid:]


def check(be, N):
    main, mid, tail = shares(be, N)
    covered = [b + j for b in main for j in (0, 1)] + mid + tail
    assert sorted(covered) == [b for b, e in enumerate(be) if e >= 0], "each expert block exactly once"
    for b in main:
        assert be[b] >= 0 and be[b + 1] == be[b], f"pair {b} is one expert's two blocks"
    nt, nt64 = (N + 255) // 256, (N + 63) // 64
    p_all, s_all = pairs_and_singles(be)
    if len(main) < len(p_all):
        assert len(main) * nt <= (len(p_all) * nt // CUS) * CUS
        assert 2 * (len(p_all) * nt % CUS) < CUS
    left = len(s_all) + 2 * (len(p_all) - len(main))
    if len(mid) < left:
        assert 2 * (left * nt % CUS) < CUS
    return main, mid, tail, nt64


def test_pairs_follow_runs():
    # runs 0x3 (a pair and a single), -1, 0x2 (a pair), 1x1, 0x1 (single again)
    be = [0, 0, 0, -1, 0, 0, 1, 0]
    assert pairs_and_singles(be) == ([0, 4], [2, 6, 7])


def test_moe_workload_split():
    """8 experts x 8192 tokens, N 4096: 68 blocks, 32 pairs and 4 single
    blocks (the odd runs' last blocks): 512 tiles of 256x256 = 2 whole rounds,
    nothing for the middle launch, the 4 singles as 128x64 tiles."""
    wl = workloads.config(4)
    be = block_experts(wl.m_indices, wl.E)
    main, mid, tail, nt64 = check(be, wl.N)
    assert (len(be), len(main), len(mid), len(tail)) == (68, 32, 0, 4)
    assert len(main) * (wl.N // 256) == 2 * CUS and len(tail) * nt64 == CUS
    assert fp8.gemm_plan("contiguous", wl.M, wl.N, wl.K)["paired"] == 1


@pytest.mark.parametrize("seed", range(40))
def test_random_layouts_cover_every_block_once(seed):
    rng = np.random.default_rng(seed)
    E = int(rng.integers(1, 12))
    be = []
    while len(be) < int(rng.integers(2, 400)):
        if rng.random() < 0.1:
            be += [-1] * int(rng.integers(1, 4))
        be += [int(rng.integers(0, E))] * int(rng.integers(1, 12))
    for N in (256, 4096, 7168):
        check(be, N)
