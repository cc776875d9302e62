"""C-ABI checks that need no GPU: the library loads, exports exactly what
include/fp8gemm.h declares, and rejects bad arguments on the host before any
device call (status codes as documented in the header)."""
import ctypes
import os
import re

import pytest

import fine_grained_block_e4m3_amd as fp8

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fp8gemm.h")

OK, INVALID, SHAPE, ALIGN, UNSUP, NODEV, LAUNCH, SCRATCH = range(8)
P = ctypes.c_void_p
A = P(4096)           # an aligned fake device address: never dereferenced on the host
MIS = P(4097)


@pytest.fixture(scope="module")
def L():
    if not os.path.exists(fp8.LIB_PATH):
        from fine_grained_block_e4m3_amd import build
        build.build()
    return fp8.load_library()


def _declared():
    text = open(HEADER).read()
    return sorted(set(re.findall(r"\b(fp8_[a-z0-9_]+)\s*\(", text)))


def test_header_declarations_match_binding():
    assert _declared() == sorted(fp8.SYMBOLS)


def test_library_exports_every_declared_symbol(L):
    for name in _declared():
        assert hasattr(L, name), f"{name} not exported"


def test_constants(L):
    assert L.fp8_get_mk_alignment_for_contiguous_layout() == 128
    for s in range(8):
        assert L.fp8_status_string(s) and L.fp8_status_string(s) != b"unknown status"
    assert L.fp8_status_string(99) == b"unknown status"


def _gemm(L, xq=A, sa=A, wq=A, sb=A, y=A, M=4, N=8, K=128, flags=0):
    return L.fp8_gemm_nt(xq, sa, wq, sb, y, M, N, K, flags, None)


def test_gemm_validation(L):
    assert _gemm(L, xq=None) == INVALID
    assert _gemm(L, y=None) == INVALID
    assert _gemm(L, M=-1) == INVALID
    assert _gemm(L, N=1 << 31) == INVALID
    assert _gemm(L, flags=4) == INVALID
    assert _gemm(L, flags=fp8.FLAG_UE8M0 | fp8.FLAG_FAST_ACCUM, M=0) == OK
    assert _gemm(L, K=100) == SHAPE
    assert _gemm(L, K=0) == SHAPE
    assert _gemm(L, xq=MIS) == ALIGN
    assert _gemm(L, y=MIS) == ALIGN
    # empty problems are a no-op, even with null pointers
    assert _gemm(L, M=0, xq=None, y=None) == OK
    assert _gemm(L, N=0) == OK


def test_quant_validation(L):
    assert L.fp8_quant_1x128(None, 4, 128, A, A, 0, None) == INVALID
    assert L.fp8_quant_1x128(A, 4, 130, A, A, 0, None) == SHAPE
    assert L.fp8_quant_1x128(MIS, 4, 128, A, A, 0, None) == ALIGN
    assert L.fp8_quant_1x128(A, 0, 128, None, None, 0, None) == OK
    assert L.fp8_quant_128x128(A, 4, 128, None, A, 0, None) == INVALID
    assert L.fp8_quant_128x128(A, 4, 64, A, A, 0, None) == SHAPE
    assert L.fp8_quant_128x128(A, 4, 128, A, A, 4, None) == INVALID


def _gpu_visible() -> bool:
    import torch
    return torch.cuda.is_available()


def test_grouped_validation(L):
    c = L.fp8_grouped_gemm_contiguous
    if not _gpu_visible():   # valid arguments: on a GPU this would launch on fake addresses
        assert c(A, A, A, A, A, A, 256, 128, 128, 2, 0, None) in (NODEV, OK, LAUNCH)
    assert c(A, A, A, A, A, A, 256, 100, 128, 2, 0, None) == SHAPE     # N % 128
    assert c(A, A, A, A, None, A, 256, 128, 128, 2, 0, None) == INVALID
    assert c(A, A, A, A, A, A, 256, 128, 128, -1, 0, None) == INVALID
    assert c(A, A, A, A, A, A, 256, 128, 128, 0, 0, None) == OK
    m = L.fp8_grouped_gemm_masked
    if not _gpu_visible():
        assert m(A, A, A, A, A, A, 4, 256, 128, 256, 0, None) in (NODEV, OK, LAUNCH)
    assert m(A, A, A, A, A, A, 4, 256, 128, 200, 0, None) == SHAPE
    assert m(A, A, A, A, A, A, 4, 256, 96, 256, 0, None) == SHAPE
    assert m(A, A, A, A, None, A, 4, 256, 128, 256, 0, None) == INVALID
    assert m(A, A, A, A, A, MIS, 4, 256, 128, 256, 0, None) == ALIGN
    assert m(A, A, A, A, A, A, 0, 256, 128, 256, 0, None) == OK


def test_qout_validation(L):
    g = L.fp8_gemm_nt_qout
    if not _gpu_visible():   # valid arguments: on a GPU this would launch on fake addresses
        assert g(A, A, A, A, A, A, 4, 256, 128, 0, None) in (NODEV, OK, LAUNCH)
    assert g(A, A, A, A, A, A, 4, 200, 128, 0, None) == SHAPE      # N % 128
    assert g(A, A, A, A, A, A, 4, 256, 100, 0, None) == SHAPE
    assert g(A, A, A, A, None, A, 4, 256, 128, 0, None) == INVALID
    assert g(A, A, A, A, A, MIS, 4, 256, 128, 0, None) == ALIGN
    assert g(A, A, A, A, A, A, 4, 256, 128, 8, None) == INVALID
    assert g(A, A, A, A, A, A, 0, 256, 128, 0, None) == OK


def test_mx_validation(L):
    q = L.fp8_quant_mx
    assert q(None, 4, 128, A, A, None) == INVALID
    assert q(A, -1, 128, A, A, None) == INVALID
    assert q(A, 4, 48, A, A, None) == SHAPE           # K % 128
    assert q(A, 4, 96, A, A, None) == SHAPE
    assert q(MIS, 4, 128, A, A, None) == ALIGN
    assert q(A, 4, 128, A, MIS, None) == ALIGN
    assert q(A, 0, 128, None, None, None) == OK
    g = L.fp8_gemm_nt_mx
    assert g(A, A, A, A, A, 4, 8, 128, 1, None) == INVALID   # no flags defined
    assert g(None, A, A, A, A, 4, 8, 128, 0, None) == INVALID
    assert g(A, A, A, A, A, 4, 8, 96, 0, None) == SHAPE      # K % 128
    assert g(A, A, A, A, A, 4, 8, 0, 0, None) == SHAPE
    assert g(A, MIS, A, A, A, 4, 8, 128, 0, None) == ALIGN
    assert g(A, A, A, A, MIS, 4, 8, 128, 0, None) == ALIGN
    assert g(A, A, A, A, A, 0, 8, 128, 0, None) == OK


def test_mxfp4_validation(L):
    q = L.fp8_quant_mxfp4
    assert q(None, 4, 128, A, A, None) == INVALID
    assert q(A, 4, 96, A, A, None) == SHAPE
    assert q(A, 4, 128, MIS, A, None) == ALIGN
    assert q(A, 0, 128, None, None, None) == OK
    g = L.fp8_gemm_nt_mx_w4
    assert g(A, A, A, A, A, 4, 8, 128, 2, None) == INVALID
    assert g(A, A, None, A, A, 4, 8, 128, 0, None) == INVALID
    assert g(A, A, A, A, A, 4, 8, 64, 0, None) == SHAPE
    assert g(A, A, MIS, A, A, 4, 8, 128, 0, None) == ALIGN
    assert g(A, A, A, A, A, 4, 0, 128, 0, None) == OK


def test_workspace_and_noalloc_validation(L):
    """The workspace variant and the no-allocation variant validate like
    fp8_gemm_nt; a workspace size needs a non-NULL, aligned workspace."""
    for fn in (lambda **k: L.fp8_gemm_nt_ws(k.get("xq", A), A, A, A, A, k.get("M", 4), 8, k.get("K", 128),
                                             k.get("flags", 0), k.get("ws", None), k.get("nb", 0), None),
               lambda **k: L.fp8_gemm_nt_noalloc(k.get("xq", A), A, A, A, A, k.get("M", 4), 8, k.get("K", 128),
                                                  k.get("flags", 0), None)):
        assert fn(xq=None) == INVALID
        assert fn(flags=8) == INVALID
        assert fn(K=64) == SHAPE
        assert fn(M=0) == OK
    assert L.fp8_gemm_nt_ws(A, A, A, A, A, 4, 8, 128, 0, None, 64, None) == INVALID
    assert L.fp8_gemm_nt_ws(A, A, A, A, A, 4, 8, 128, 0, MIS, 64, None) == ALIGN
    assert L.fp8_gemm_workspace_size(4, 8, 100, 0) == 0


def _plan(layout, M, N, K, flags=0, cus=256, ws=0):
    plan = fp8.GemmPlan()
    st = fp8.load_library().fp8_gemm_plan(layout, M, N, K, flags, cus, ws, ctypes.byref(plan))
    assert st == OK, st
    return plan


def test_plan_pins_the_pages_unaligned_block_example(L):
    """DeepGEMM page, section "非对齐块大小": M = 256, N = 7168 on 132 SMs gives
    112 tiles of 128x128, one wave that leaves 20 SMs idle.  The FP8-instruction
    planner takes exactly that tiling for this shape and that SM count."""
    p = _plan(0, 256, 7168, 7168, fp8.FLAG_FAST_ACCUM, cus=132)
    assert (p.tile_m, p.tile_n, p.tiles, p.grid) == (128, 128, 112, 112)
    assert 132 - p.grid == 20
    # the page's alternative, 128x112, would give 2 * 64 = 128 tiles: 97% of 132
    assert ((256 + 127) // 128) * ((7168 + 111) // 112) == 128


def test_plan_fills_whole_waves_on_the_prefill_shape(L):
    """4096x7168 on 256 CUs: 256x256 tiles are 448 = 1.75 waves; the FP8
    planner takes 256x224 (512 tiles = 2 whole waves, the same trade as the
    page's 112-wide blocks); the exact path (whose 32x32 subtiles do not
    split 224 columns over two waves) runs the columns [0, 4096) as 256 tiles
    of 256 and [4096, 7168) as 256 tiles of 192: one whole wave each."""
    f = _plan(0, 4096, 7168, 7168, fp8.FLAG_FAST_ACCUM)
    assert (f.exact, f.tile_m, f.tile_n, f.tiles, f.grid) == (0, 256, 224, 512, 256)
    e = _plan(0, 4096, 7168, 7168)
    assert (e.exact, e.tile_m, e.tile_n, e.tiles, e.waves, e.grid) == (1, 256, 256, 256, 8, 256)
    assert (e.main_cols, e.tail_tile_m, e.tail_tile_n, e.tail_tiles) == (4096, 256, 192, 256)
    assert e.main_cols + 192 * (e.tail_tiles // 16) == 7168          # the two launches tile [0, N) once
    d = _plan(0, 32, 24576, 1536)                   # exact decode kernel, X in chunks: 96 columns per workgroup
    assert (d.exact, d.kernel, d.tile_n, d.tiles, d.grid, d.k_splits) == (1, 3, 96, 256, 256, 1)
    d = _plan(0, 16, 7168, 2048)                    # fewer column tiles than CUs: X resident
    assert (d.kernel, d.tiles, d.k_splits) == (4, 75, 1)
    d = _plan(0, 64, 24576, 1536)                   # unsplit, M > 32: the 64x96 tile
    assert (d.kernel, d.tile_m, d.tile_n) == (0, 64, 96)
    assert _plan(0, 32, 4096, 3072).kernel == 4 and _plan(0, 32, 4096, 3200).kernel == 3     # 25 blocks: chunks
    assert _plan(0, 32, 24576, 3072).kernel == 3
    assert _plan(0, 65, 24576, 1536).kernel == 0
    assert _plan(0, 16, 24576, 1536, fp8.FLAG_FAST_ACCUM).kernel == 1
    assert _plan(0, 40, 24576, 1536, fp8.FLAG_FAST_ACCUM).kernel == 2
    assert _plan(0, 4096, 7168, 7168, fp8.PLAN_MX).tile_n == 224
    assert (_plan(0, 4096, 7168, 7168, fp8.PLAN_QOUT).tile_n, _plan(0, 128, 256, 512, fp8.PLAN_QOUT).tile_m) == (256, 128)


def test_plan_exact_column_split_rule(L):
    """The default path's column split: only when the two launches take fewer
    rounds' worth of tile width than 256x256 tiles throughout; the main
    launch covers whole 256-column tiles, the tail the rest of [0, N)."""
    def rounds_width(M, N, cus, cols):
        mt = -(-M // 256)
        if cols == 0:
            return -(-mt * -(-N // 256) // cus) * 256
        return -(-mt * (cols // 256) // cus) * 256 + -(-mt * -(-(N - cols) // 192) // cus) * 192
    for M, N, cus in [(4096, 7168, 256), (1900, 8102, 256), (2500, 7050, 256), (4096, 4096, 256),
                      (8192, 7168, 256), (4096, 7168, 304), (3000, 5000, 128)]:
        p = _plan(0, M, N, 7168, cus=cus)
        if p.tile_m != 256 or p.exact != 1:
            continue
        cols = p.main_cols if p.main_cols < N else 0
        assert cols % 256 == 0 and cols < N
        best = min(rounds_width(M, N, cus, c) for c in range(0, N, 256))
        assert rounds_width(M, N, cus, cols) == best
        if cols:
            assert (p.tail_tile_n, p.tail_tiles) == (192, -(-M // 256) * -(-(N - cols) // 192))
        else:
            assert p.tail_tiles == 0
    assert _plan(0, 1900, 8102, 640).main_cols == 8102       # one whole wave already: no split
    assert _plan(0, 2500, 7050, 640).main_cols == 6400       # 250 + 40 tiles: one wave each


def test_plan_masked_default_path_launches_one_workgroup_per_tile(L):
    """Masked layout, both paths: 256-row tiles of 8 waves, one workgroup
    per possible tile of an expert (the kernels skip the subtiles past the
    expert's count and the hardware dispatcher balances the unequal tiles)."""
    e = _plan(2, 256, 7168, 2048)
    assert (e.exact, e.kernel, e.tile_m, e.tile_n, e.waves, e.tiles, e.grid) == (1, 0, 256, 256, 8, 28, 28)
    e = _plan(2, 512, 7168, 2048, cus=16)
    assert (e.tiles, e.grid) == (56, 56)
    f = _plan(2, 256, 7168, 2048, fp8.FLAG_FAST_ACCUM, cus=16)
    assert (f.exact, f.tile_m, f.tile_n, f.tiles, f.grid) == (0, 256, 256, 28, 28)


@pytest.mark.parametrize("fast", [0, fp8.FLAG_FAST_ACCUM])
@pytest.mark.parametrize("M", [128, 8704, 9216, 1088 * 128 // 16, 33 * 128, 256 * 128 + 128])
def test_plan_contiguous_launches_cover_every_row_once(L, M, fast):
    """Contiguous layout: 128-row tiles; when the last round of 128x256 tiles
    would leave over half of the CUs idle, the blocks past the full rounds go
    to a second launch of smaller tiles.  The two launches cover [0, M)
    exactly once, at whole 128-row blocks, and the first holds whole rounds."""
    N, cus = 4096, 256
    p = _plan(1, M, N, 7168, fast)
    if p.paired:
        # the pair schedule (test_plan_contiguous_pair_schedule)
        assert M > 128
        return
    assert p.tile_m == 128 and p.tile_n == 256
    assert p.main_rows % 128 == 0 and 0 < p.main_rows <= M
    assert p.tiles == ((p.main_rows + 127) // 128) * (N // 256)
    if p.main_rows < M:
        assert p.tiles % cus == 0, "the first launch holds whole rounds"
        assert p.tail_tile_m == 128 and p.tail_tile_n in (64, 128)
        assert p.tail_tiles == ((M - p.main_rows + 127) // 128) * (N // p.tail_tile_n)
        blocks = ((M + 127) // 128) * (N // 256)
        assert 2 * (blocks % cus) < cus
    else:
        assert p.tail_tile_m == 0


@pytest.mark.parametrize("fast", [0, fp8.FLAG_FAST_ACCUM])
@pytest.mark.parametrize("M", [8704, 33 * 128, 1024 * 128])
def test_plan_contiguous_pair_schedule(L, M, fast):
    """Contiguous layout, at least a round of 256x256 tiles if every 128-row
    block were paired: three launches, 256x256 tiles over the pairs of one
    expert's blocks, then 128x256 and 128x64 tiles over the blocks left,
    their shares found on the device (upper bounds here)."""
    N, cus = 4096, 256
    p = _plan(1, M, N, 7168, fast)
    assert p.paired == 1 and p.exact == (0 if fast else 1)
    assert (p.tile_m, p.tile_n, p.waves, p.main_rows) == (256, 256, 8, M)
    assert p.tiles == (M + 255) // 256 * (N // 256) and p.grid == min(p.tiles, cus)
    assert (p.mid_tile_m, p.mid_tile_n, p.mid_tiles) == (128, 256, (M + 127) // 128 * (N // 256))
    assert (p.tail_tile_m, p.tail_tile_n, p.tail_tiles) == (128, 64, (M + 127) // 128 * (N // 64))


@pytest.mark.parametrize("M,N,flags", [(1024 * 128 + 1, 4096, 0), (4096 - 256, 4096, 0), (8704, 256, 0),
                                       (1024 * 128 + 1, 4096, fp8.FLAG_FAST_ACCUM)])
def test_plan_contiguous_unpaired(L, M, N, flags):
    """No pair schedule past 1024 blocks of 128 rows (its LDS table) or
    below a round of 256x256 tiles."""
    p = _plan(1, M, N, 7168, flags)
    assert p.paired == 0 and p.tile_m == 128 and (p.mid_tile_m, p.mid_tiles) == (0, 0)


def test_plan_decode_split_and_workspace(L):
    """The decode kernel splits K over workgroups only with a workspace that
    holds the partial sums: 16 x 2112 x 7168 on 256 CUs, 22 column tiles of 96,
    at most 8 splits."""
    p0 = _plan(0, 16, 2112, 7168, fp8.FLAG_FAST_ACCUM, ws=0)
    assert (p0.kernel, p0.k_splits, p0.workspace_bytes, p0.tiles) == (1, 1, 0, 22)
    big = 1 << 30
    p = _plan(0, 16, 2112, 7168, fp8.FLAG_FAST_ACCUM, ws=big)
    assert p.k_splits == 8 and p.workspace_bytes == 8 * 16 * 2112 * 4 and p.tiles == 22 * 8
    p2 = _plan(0, 16, 2112, 7168, fp8.FLAG_FAST_ACCUM, ws=p.workspace_bytes - 1)
    assert p2.k_splits == 1
    e = _plan(0, 16, 2112, 7168, 0, ws=big)       # exact decode kernel: 96-column tiles
    assert (e.kernel, e.k_splits, e.tiles, e.workspace_bytes) == (4, 8, 22 * 8, 8 * 16 * 2112 * 4)
    e = _plan(0, 64, 4096, 7168, 0, ws=big)       # 43 tiles: 256 // 43 = 5 splits of 11-12 blocks
    assert (e.kernel, e.k_splits, e.workspace_bytes) == (4, 5, 5 * 64 * 4096 * 4)
    e = _plan(0, 64, 4096, 7168, 0, ws=0)         # no workspace, M > 32: the 64x96 tile
    assert (e.kernel, e.k_splits, e.workspace_bytes) == (0, 1, 0)
    e = _plan(0, 16, 4096, 7168, 0, ws=0)         # no workspace, M <= 32: one range of 56 blocks, X in chunks
    assert (e.kernel, e.k_splits, e.workspace_bytes) == (3, 1, 0)
    e = _plan(0, 16, 2112, 32768, 0, ws=big)      # 8 ranges of 32 blocks: X in chunks, split
    assert (e.kernel, e.k_splits) == (3, 8)
    # the largest split a 256-CU device asks for fits the no-allocation entry point's 8 MiB
    worst = max(_plan(0, 64, n, 7168, 0, ws=big).workspace_bytes for n in range(96, 96 * 129, 96))
    assert 0 < worst <= 64 * 4 * 96 * 256 <= 8 << 20
    assert _plan(0, 64, 24576, 1536, 0, ws=big).k_splits == 1     # 256 tiles: no split


def test_plan_validation(L):
    plan = fp8.GemmPlan()
    f = L.fp8_gemm_plan
    assert f(3, 4, 8, 128, 0, 256, 0, ctypes.byref(plan)) == INVALID
    assert f(0, 4, 8, 128, 0, 0, 0, ctypes.byref(plan)) == INVALID
    assert f(0, 4, 8, 128, 0, 256, 0, None) == INVALID
    assert f(1, 4, 8, 128, fp8.PLAN_MX, 256, 0, ctypes.byref(plan)) == INVALID
    assert f(0, 4, 8, 100, 0, 256, 0, ctypes.byref(plan)) == SHAPE


def test_no_device_reported_without_gpu(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _gemm(L) == NODEV
    assert L.fp8_gemm_nt_noalloc(A, A, A, A, A, 4, 8, 128, 0, None) == NODEV
    assert L.fp8_gemm_workspace_size(16, 2112, 7168, fp8.FLAG_FAST_ACCUM) == 0
    assert L.fp8_quant_1x128(A, 4, 128, A, A, 0, None) == NODEV
    assert L.fp8_quant_mx(A, 4, 128, A, A, None) == NODEV
    assert L.fp8_gemm_nt_mx(A, A, A, A, A, 4, 8, 128, 0, None) == NODEV
    assert L.fp8_quant_mxfp4(A, 4, 128, A, A, None) == NODEV
    assert L.fp8_gemm_nt_mx_w4(A, A, A, A, A, 4, 8, 128, 0, None) == NODEV


def test_binding_refuses_cpu_tensors():
    import torch
    x = torch.zeros(4, 128)
    with pytest.raises(ValueError, match="GPU tensor"):
        fp8.quant_1x128(x)


def test_library_imports_no_allocation_or_synchronization():
    """The library allocates, frees and synchronizes nothing: none of the HIP
    runtime's allocation, free, copy, fill or synchronization routines is
    among the symbols it imports (read from the built shared object)."""
    import shutil
    import subprocess
    nm = shutil.which("nm")
    if nm is None:
        pytest.skip("nm not available")
    out = subprocess.run([nm, "-D", "--undefined-only", fp8.LIB_PATH], capture_output=True, text=True,
                         check=True).stdout
    imported = {line.split()[-1].split("@")[0] for line in out.splitlines() if line.strip()}
    hip = sorted(s for s in imported if s.startswith("hip"))
    assert "hipLaunchKernel" in hip, hip
    forbidden = ("Malloc", "Free", "Memcpy", "Memset", "Synchronize", "HostRegister", "MallocAsync")
    bad = [s for s in hip if any(f in s for f in forbidden)]
    assert not bad, bad
