"""GPU grouped (MoE) GEMMs against the oracle.  Row handling is bit-exact:
every row the oracle leaves unwritten must keep its sentinel bits.  Values
follow the same two-path rule as the dense tests (default, exact partials:
the tolerance everywhere; FP8_FLAG_FAST_ACCUM: the tolerance on the headline
workloads, elsewhere the tolerance or the measured truncation-model bound,
with a ceiling on the elements outside the tolerance)."""
import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import (SENTINEL, assert_close, assert_close_or_bounded, bf16_bits, dev,
                         fp8_mfma_error_bound, say, sentinel_like)

pytestmark = pytest.mark.gpu
PATHS = [pytest.param(False, id="exact"), pytest.param(True, id="fast")]


def quant(wl):
    flags = oracle.FLAG_UE8M0 if wl.ue8m0 else 0
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    return xq, sa, wq, sb, flags


def run_contiguous(xq, sa, wq, sb, idx, E, flags, fast):
    M, K = xq.shape
    N = wq.shape[0] // E
    say(f"contiguous M={M} N={N} K={K} E={E} flags={flags} fast_accum={fast}")
    y = sentinel_like((M, N))
    fp8.grouped_gemm_contiguous(dev(xq), dev(sa), dev(wq.reshape(E, N, K)),
                                dev(sb.reshape(E, N // 128, K // 128)),
                                dev(idx.astype(np.int32)), ue8m0=bool(flags), fast_accum=fast,
                                out=y)
    return bf16_bits(y)


def run_masked(xq, sa, wq, sb, mm, E, max_m, flags, fast):
    MT, K = xq.shape
    N = wq.shape[0] // E
    say(f"masked E={E} max_m={max_m} N={N} K={K} counts={list(mm)} flags={flags} "
        f"fast_accum={fast}")
    y = sentinel_like((E, max_m, N))
    fp8.grouped_gemm_masked(dev(xq.reshape(E, max_m, K)), dev(sa), dev(wq.reshape(E, N, K)),
                            dev(sb.reshape(E, N // 128, K // 128)), dev(mm.astype(np.int32)),
                            ue8m0=bool(flags), fast_accum=fast, out=y)
    return bf16_bits(y).reshape(E * max_m, N)


def grouped_bound(xq, sa, wq, sb, ref, row_expert, E, pow2):
    """FP8-MFMA model bound, row by row with each row's own expert weights."""
    N = wq.shape[0] // E
    NB = N // 128
    bound = np.zeros_like(ref)
    for e in range(E):
        rows = np.nonzero(row_expert == e)[0]
        if len(rows):
            bound[rows] = fp8_mfma_error_bound(xq[rows], np.ascontiguousarray(sa[:, rows]),
                                               wq[e * N:(e + 1) * N], sb[e * NB:(e + 1) * NB],
                                               ref[rows], pow2=pow2)
    return bound


def check_rows(y, ref, written, what, bound=None):
    assert np.all(y[~written] == SENTINEL), f"{what}: a row outside the valid set was written"
    if not written.any():
        return
    if bound is None:
        say(f"stats {assert_close(y[written], ref[written], what)}")
    else:
        say(f"stats {assert_close_or_bounded(y[written], ref[written], bound[written], what)}")


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("counts", [[0, 130, 1, 169], [500, 0, 0, 0], [1, 1, 1, 1],
                                    [128, 256, 0, 7]])
def test_contiguous_routing(counts, fast):
    wl = workloads.contiguous(E=4, tokens=sum(counts), N=256, K=384, seed=sum(counts),
                              counts=np.array(counts))
    xq, sa, wq, sb, flags = quant(wl)
    ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E)
    y = run_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E, flags, fast)
    bound = None if not fast else grouped_bound(xq, sa, wq, sb, ref,
                                               np.where(written, wl.m_indices, -1), wl.E, False)
    check_rows(y, ref, written, f"contiguous {counts}", bound)


@pytest.mark.parametrize("fast", PATHS)
def test_contiguous_tail_blocks_in_a_second_launch(fast):
    """18 row blocks x 16 column tiles of 128x256 = 288 tiles: on 256 CUs one
    full round, then the last 2 row blocks (part of expert 3 and its padding
    rows) run as a second launch of 128x64 tiles."""
    counts = [500, 600, 700, 300]
    wl = workloads.contiguous(E=4, tokens=sum(counts), N=4096, K=256, seed=77,
                              counts=np.array(counts))
    assert wl.M == 18 * 128
    xq, sa, wq, sb, flags = quant(wl)
    ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E)
    y = run_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E, flags, fast)
    bound = None if not fast else grouped_bound(xq, sa, wq, sb, ref,
                                               np.where(written, wl.m_indices, -1), wl.E, False)
    check_rows(y, ref, written, "contiguous tail launch", bound)


@pytest.mark.parametrize("fast", PATHS)
def test_contiguous_dirichlet_and_bad_indices(fast):
    wl = workloads.contiguous(E=8, tokens=1500, N=384, K=256, seed=41)
    idx = wl.m_indices.copy()
    # contract violations, defined as "skip": out-of-range experts and a
    # foreign expert inside another expert's aligned block
    idx[idx == 3] = 99
    first5 = np.nonzero(idx == 5)[0]
    if len(first5) > 3:
        idx[first5[1:3]] = 6
    xq, sa, wq, sb, flags = quant(wl)
    ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, idx, wl.E)
    y = run_contiguous(xq, sa, wq, sb, idx, wl.E, flags, fast)
    bound = None if not fast else grouped_bound(xq, sa, wq, sb, ref,
                                               np.where(written, idx, -1), wl.E, False)
    check_rows(y, ref, written, "contiguous dirichlet", bound)


def block_layout(block_experts, seed):
    """Row indices of 128-row blocks: block i belongs to expert
    block_experts[i] (-1: a block of padding rows only); the last block of
    each run of one expert keeps a random number of its rows (at least one)
    and pads the rest with -1, as the layout pads an expert's rows up to the
    alignment."""
    rng = np.random.default_rng(seed)
    be = np.asarray(block_experts)
    idx = np.repeat(be, 128).astype(np.int32)
    for i, e in enumerate(be):
        if e >= 0 and (i + 1 == len(be) or be[i + 1] != e):
            idx[i * 128 + int(rng.integers(1, 129)):(i + 1) * 128] = -1
    return idx


# Block layouts for the pair schedule (256x256 tiles over pairs of one
# expert's consecutive blocks, then 128x256 and 128x64 tiles over the blocks
# left; N = 4096, 256 CUs: 16 pairs or blocks per round).
PAIR_LAYOUTS = {
    # 17 pairs = 272 tiles of 256x256: the first launch keeps one round and
    # passes the 17th pair on; 16 singles + its 2 blocks = 288 tiles of
    # 128x256: the second keeps one round, the third takes 2 blocks
    "passed_on": [0] * 34 + list(range(1, 17)),
    # runs across the 64-block chunks in which the schedule is built: block
    # 64 is the second block of a pair
    "chunk_carry": [0] + [1] * 70 + [2] * 29,
    # runs broken by padding blocks, one expert in two runs, runs of odd length
    "breaks": [0] * 3 + [-1] + [0] * 2 + [1] * 5 + [2] + [1] * 9 + [-1, -1] + [3] * 11 + [4],
    # no two consecutive blocks of one expert: every block single
    "all_single": [0, 1] * 20,
    # M not a multiple of 128: the last pair's second block holds 50 rows
    "ragged_end": [0] * 33 + [1] * 4,
    # 3 pairs = 48 tiles: the first launch keeps none; 11 singles + 6 pair
    # blocks = 272 tiles of 128x256: the second keeps 16 blocks, the third
    # takes the last pair block; padding-only blocks in no launch
    "mid_and_tail": [0, 0, 1, 1, 2, 2] + list(range(3, 14)) + [-1] * 14,
}
PAIR_ROWS = {"ragged_end": 36 * 128 + 50}


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("layout,flags", [(name, 0) for name in PAIR_LAYOUTS]
                         + [("passed_on", oracle.FLAG_UE8M0), ("breaks", oracle.FLAG_UE8M0)])
def test_contiguous_pair_schedule(layout, flags, fast):
    """The pair schedule on layouts that exercise each of its branches, with
    FP32 scales and, on two layouts, power-of-two scales (the UE8M0 kernel
    instances)."""
    blocks = PAIR_LAYOUTS[layout]
    idx = block_layout(blocks, seed=len(blocks))[:PAIR_ROWS.get(layout)]
    E, N, K = max(blocks) + 1, 4096, 256 if flags else 128
    plan = fp8.gemm_plan("contiguous", len(idx), N, K, ue8m0=bool(flags), fast_accum=fast)
    assert plan["paired"] == 1
    wl = workloads.dense(len(idx), N * E, K, seed=23)
    xq, sa = oracle.quant_1x128(wl.x, flags)
    wq, sb = oracle.quant_128x128(wl.w, flags)
    ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, idx, E, flags)
    assert np.array_equal(written, idx >= 0)
    y = run_contiguous(xq, sa, wq, sb, idx, E, flags, fast)
    bound = None if not fast else grouped_bound(xq, sa, wq, sb, ref, idx, E, bool(flags))
    check_rows(y, ref, written, f"contiguous pairs {layout} flags={flags}", bound)


def random_block_experts(rng, E):
    """A random block layout of 32 to 120 blocks: runs of 1 to 9 blocks of a
    random expert (an expert may recur, a neighbour may repeat it, so runs
    merge), with padding-only blocks (-1) between some runs."""
    out = []
    while len(out) < 32 or (len(out) < 120 and rng.random() < 0.9):
        if out and rng.random() < 0.15:
            out += [-1] * int(rng.integers(1, 3))
        out += [int(rng.integers(0, E))] * int(rng.integers(1, 10))
    return out[:120]


@pytest.mark.parametrize("fast", PATHS)
def test_contiguous_pair_schedule_random_layouts(fast):
    """Twelve random block layouts through the pair schedule (each paired
    by the planner, N = 4096), every row against the oracle."""
    rng = np.random.default_rng(2024)
    N, K, E = 4096, 128, 6
    wl = workloads.dense(120 * 128, N * E, K, seed=31)
    xq_all, sa_all = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    for case in range(12):
        blocks = random_block_experts(rng, E)
        idx = block_layout(blocks, seed=case)
        M = len(idx)
        assert fp8.gemm_plan("contiguous", M, N, K, fast_accum=fast)["paired"] == 1
        xq, sa = xq_all[:M], np.ascontiguousarray(sa_all[:, :M])
        say(f"case {case}: {len(blocks)} blocks {blocks}")
        ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, idx, E)
        y = run_contiguous(xq, sa, wq, sb, idx, E, 0, fast)
        bound = None if not fast else grouped_bound(xq, sa, wq, sb, ref, np.where(written, idx, -1), E, False)
        check_rows(y, ref, written, f"contiguous pairs, random layout {case}", bound)


@pytest.mark.parametrize("fast", PATHS)
def test_contiguous_pair_schedule_graph_replays(fast):
    """The three launches of the pair schedule captured in a graph: every
    replay, with eager work and synchronizations between replays, equals the
    eager result bit for bit; and since every workgroup rebuilds the schedule
    from the row indices, a replay after new indices are written into the
    same buffer follows them."""
    blocks = PAIR_LAYOUTS["passed_on"]
    idx = block_layout(blocks, seed=5)
    E, N, K = max(blocks) + 1, 4096, 128
    wl = workloads.dense(len(idx), N * E, K, seed=29)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    ops = (dev(xq), dev(sa), dev(wq.reshape(E, N, K)), dev(sb.reshape(E, N // 128, K // 128)))
    d_idx = dev(idx)
    y = sentinel_like((len(idx), N))
    s = torch.cuda.Stream()
    run = lambda: fp8.grouped_gemm_contiguous(*ops, d_idx, fast_accum=fast, out=y)
    with torch.cuda.stream(s):
        run()
    torch.cuda.synchronize()
    eager = bf16_bits(y)
    g = torch.cuda.CUDAGraph()
    say(f"contiguous pairs: capture fast_accum={fast}")
    with torch.cuda.graph(g, stream=s):
        run()
    for i in range(3):
        y.view(torch.int16).fill_(SENTINEL)
        torch.cuda.synchronize()
        g.replay()
        fp8.grouped_gemm_contiguous(*ops, d_idx, fast_accum=not fast)   # eager work between replays
        torch.cuda.synchronize()
        assert np.array_equal(bf16_bits(y), eager), f"replay {i}"
    # other row indices in the same buffer (runs broken by padding blocks)
    idx2 = np.resize(block_layout(PAIR_LAYOUTS["breaks"], seed=6), len(idx)).astype(np.int32)
    d_idx.copy_(dev(idx2))
    y.view(torch.int16).fill_(SENTINEL)
    torch.cuda.synchronize()
    g.replay()
    torch.cuda.synchronize()
    ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, idx2, E)
    bound = None if not fast else grouped_bound(xq, sa, wq, sb, ref, np.where(written, idx2, -1), E, False)
    check_rows(bf16_bits(y), ref, written, "contiguous pairs, replay with new indices", bound)


@pytest.mark.parametrize("fast", PATHS)
def test_contiguous_ue8m0(fast):
    wl = workloads.contiguous(E=3, tokens=400, N=256, K=256, seed=42)
    xq, sa = oracle.quant_1x128(wl.x, oracle.FLAG_UE8M0)
    wq, sb = oracle.quant_128x128(wl.w, oracle.FLAG_UE8M0)
    ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E,
                                             oracle.FLAG_UE8M0)
    y = run_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E, oracle.FLAG_UE8M0, fast)
    bound = None if not fast else grouped_bound(xq, sa, wq, sb, ref,
                                               np.where(written, wl.m_indices, -1), wl.E, True)
    check_rows(y, ref, written, "contiguous ue8m0", bound)


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("ue8m0", [True, False])
@pytest.mark.parametrize("max_m", [200, 256, 300])
def test_masked_counts(ue8m0, max_m, fast):
    mm = np.array([0, 1, 127, 128, 255, 256, -3, 999], np.int32)
    E = len(mm)
    wl = workloads.masked(E, max_m, 256, 384, seed=max_m, ue8m0=ue8m0, masked_m=mm)
    xq, sa, wq, sb, flags = quant(wl)
    ref, written = oracle.grouped_masked(xq, sa, wq, sb, mm, E, max_m, flags)
    y = run_masked(xq, sa, wq, sb, mm, E, max_m, flags, fast)
    bound = None
    if fast:
        row_expert = np.where(written, np.arange(E * max_m) // max_m, -1)
        bound = grouped_bound(xq, sa, wq, sb, ref, row_expert, E, ue8m0)
    check_rows(y, ref, written, f"masked max_m={max_m}", bound)


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("ue8m0", [True, False])
def test_masked_tile_order(ue8m0, fast):
    """Experts with one, two and three 128-row m-tiles (and none) times three
    256-column n-tiles, the last one ragged: the tile order walks each
    expert's m-tiles fastest within each n-tile; every valid row of every
    column is written once and nothing else."""
    mm = np.array([300, 129, 0, 257, 64], np.int32)
    E, max_m, N, K = len(mm), 300, 640, 256
    wl = workloads.masked(E, max_m, N, K, seed=11, ue8m0=ue8m0, masked_m=mm)
    xq, sa, wq, sb, flags = quant(wl)
    ref, written = oracle.grouped_masked(xq, sa, wq, sb, mm, E, max_m, flags)
    y = run_masked(xq, sa, wq, sb, mm, E, max_m, flags, fast)
    row_expert = np.where(written, np.arange(E * max_m) // max_m, -1)
    bound = grouped_bound(xq, sa, wq, sb, ref, row_expert, E, ue8m0) if fast else None
    check_rows(y, ref, written, "masked tile order", bound)


@pytest.mark.parametrize("fast", PATHS)
@pytest.mark.parametrize("E", [63, 64, 65, 90])
def test_masked_many_experts(E, fast):
    """Expert counts around 64 (the default path walks up to 64 experts
    largest first, more in expert order), with equal counts among them (ties
    walk in expert order) and empty experts: every valid row of every
    expert is written once, with the right expert's weights, and nothing
    else."""
    rng = np.random.default_rng(E)
    mm = rng.integers(0, 70, E).astype(np.int32)
    mm[::7] = 33                                    # ties
    mm[3::11] = 0                                   # empty experts
    max_m, N, K = 64, 256, 256
    wl = workloads.masked(E, max_m, N, K, seed=E, ue8m0=False, masked_m=mm)
    xq, sa, wq, sb, flags = quant(wl)
    ref, written = oracle.grouped_masked(xq, sa, wq, sb, mm, E, max_m, flags)
    y = run_masked(xq, sa, wq, sb, mm, E, max_m, flags, fast)
    row_expert = np.where(written, np.arange(E * max_m) // max_m, -1)
    bound = grouped_bound(xq, sa, wq, sb, ref, row_expert, E, False) if fast else None
    check_rows(y, ref, written, f"masked E={E}", bound)


@pytest.mark.parametrize("fast", PATHS)
def test_masked_rows_past_count_never_read(fast):
    """Rows past the count may hold NaN codes and NaN scales: the output must
    not change."""
    E, max_m, N, K = 3, 256, 256, 256
    mm = np.array([5, 0, 200], np.int32)
    wl = workloads.masked(E, max_m, N, K, seed=3, masked_m=mm)
    xq, sa, wq, sb, flags = quant(wl)
    y0 = run_masked(xq, sa, wq, sb, mm, E, max_m, flags, fast)
    xq2 = xq.copy()
    sa2 = sa.copy()
    for e in range(E):
        xq2[e * max_m + mm[e]:(e + 1) * max_m] = 0x7F      # NaN codes
        sa2[:, e * max_m + mm[e]:(e + 1) * max_m] = np.nan
    y1 = run_masked(xq2, sa2, wq, sb, mm, E, max_m, flags, fast)
    assert np.array_equal(y0, y1)


@pytest.mark.slow
@pytest.mark.parametrize("fast", PATHS)
def test_full_size_contiguous_config4_every_element(fast):
    wl = workloads.config(4)
    say("config 4: oracle quantization")
    xq, sa, wq, sb, flags = quant(wl)
    y = run_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E, flags, fast)
    say("config 4: oracle grouped GEMM")
    ref, written = oracle.grouped_contiguous(xq, sa, wq, sb, wl.m_indices, wl.E)
    assert np.array_equal(written, wl.m_indices >= 0)
    check_rows(y, ref, written, "config 4")


@pytest.mark.slow
@pytest.mark.parametrize("fast", PATHS)
def test_full_size_masked_config5_every_element(fast):
    wl = workloads.config(5)
    say("config 5: oracle quantization")
    xq, sa, wq, sb, flags = quant(wl)
    E, max_m = wl.E, wl.max_m
    y = run_masked(xq, sa, wq, sb, wl.masked_m, E, max_m, flags, fast)
    say("config 5: oracle grouped GEMM")
    ref, written = oracle.grouped_masked(xq, sa, wq, sb, wl.masked_m, E, max_m, flags)
    check_rows(y, ref, written, "config 5")


def test_nothing_to_compute():
    """Calls with no valid row launch nothing or exit at once and write
    nothing: every masked count zero (or negative), every contiguous row
    index padding or out of range, and a dense call with M = 0."""
    E, max_m, N, K = 3, 128, 256, 256
    mm = np.array([0, -5, 0], np.int32)
    wl = workloads.masked(E, max_m, N, K, seed=21, masked_m=mm)
    xq, sa, wq, sb, flags = quant(wl)
    y = run_masked(xq, sa, wq, sb, mm, E, max_m, flags, False)
    assert np.all(y == SENTINEL)
    idx = np.array([-1] * 128 + [E] * 128 + [-7] * 128, np.int32)
    wl = workloads.dense(len(idx), N * E, K, seed=22)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    y = run_contiguous(xq, sa, wq, sb, idx, E, 0, False)
    assert np.all(y == SENTINEL)
    say("dense M = 0")
    z = fp8.gemm_nt(torch.empty((0, K), dtype=torch.uint8, device="cuda"),
                    torch.empty((K // 128, 0), dtype=torch.float32, device="cuda"),
                    dev(wq[:N]), dev(sb[:N // 128]))
    torch.cuda.synchronize()
    assert tuple(z.shape) == (0, N)
