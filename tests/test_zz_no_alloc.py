"""fp8_gemm_nt_noalloc (the entry point that allocates nothing: its split-K
partial sums live in the library's fixed device array) against
fp8_gemm_nt_ws, the entry point whose caller-owned workspace it replaces,
called through the C ABI.  Calls in a row on decode shapes that split K, on
the default path and with FP8_FLAG_FAST_ACCUM, each smaller than the one
before, so that a call reads nothing the one before left behind; the first
default-path shape needs more than 4 MiB of the array.  The outputs must be
bit-identical (same kernels, same split, same summation order), and nothing
outside the output may be written."""
import ctypes

import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import bf16_bits, check_guards, dev, guarded, say

pytestmark = pytest.mark.gpu


def _ptr(t):
    return ctypes.c_void_p(t.data_ptr())


def _call(L, name, a, y, M, N, K, flags, ws=None):
    s = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    if name == "fp8_gemm_nt_ws":
        st = L.fp8_gemm_nt_ws(*[_ptr(t) for t in a], _ptr(y), M, N, K, flags,
                              _ptr(ws) if ws is not None else None, ws.numel() if ws is not None else 0, s)
    else:
        st = getattr(L, name)(*[_ptr(t) for t in a], _ptr(y), M, N, K, flags, s)
    assert st == 0, (name, fp8.STATUS.get(st, st))


@pytest.mark.parametrize("flags", [fp8.FLAG_FAST_ACCUM, 0])
def test_noalloc_equals_the_workspace_entry_point(flags):
    L = fp8.load_library()
    shapes = [(16, 2112, 7168), (8, 1000, 2176)]
    if not flags & fp8.FLAG_FAST_ACCUM:
        shapes = [(64, 4096, 7168)] + shapes
    for M, N, K in shapes:
        wl = workloads.dense(M, N, K, seed=M + N, outlier_frac=0.01, outlier_mult=50.0)
        xq, sa = oracle.quant_1x128(wl.x)
        wq, sb = oracle.quant_128x128(wl.w)
        a = [dev(t) for t in (xq, sa, wq, sb)]
        need = L.fp8_gemm_workspace_size(M, N, K, flags)
        assert need > 0, "the case must split K"
        if M == 64:
            assert need > 4 << 20
        say(f"noalloc M={M} N={N} K={K} flags={flags} scratch bytes={need}")
        ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
        full_ws, y_ws = guarded((M, N))
        full_na, y_na = guarded((M, N))
        _call(L, "fp8_gemm_nt_ws", a, y_ws, M, N, K, flags, ws if need else None)
        _call(L, "fp8_gemm_nt_noalloc", a, y_na, M, N, K, flags)
        torch.cuda.synchronize()
        check_guards(full_ws, M * N)
        check_guards(full_na, M * N)
        assert np.array_equal(bf16_bits(y_na), bf16_bits(y_ws)), f"M={M} N={N} K={K}"
