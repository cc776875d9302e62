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

OK, INVALID, SHAPE, ALIGN, UNSUP, NODEV, LAUNCH = range(7)
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
    for s in range(7):
        assert L.fp8_status_string(s)
    assert L.fp8_status_string(99) == b"unknown status"


def _gemm(L, xq=A, sa=A, wq=A, sb=A, y=A, M=4, N=8, K=128, flags=0):
    return L.fp8_gemm_nt(xq, sa, wq, sb, y, M, N, K, flags, None)


def test_gemm_validation(L):
    assert _gemm(L, xq=None) == INVALID
    assert _gemm(L, y=None) == INVALID
    assert _gemm(L, M=-1) == INVALID
    assert _gemm(L, N=1 << 31) == INVALID
    assert _gemm(L, flags=4) == INVALID
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


def test_no_device_reported_without_gpu(L):
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is visible")
    assert _gemm(L) == NODEV
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
