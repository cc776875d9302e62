"""Plain CPU oracle for the fine-grained block-scaled E4M3 GEMM.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py`` may import this package.  The GPU product path
(``fine_grained_block_e4m3_amd``) never imports it and shares no code with it.

The arithmetic lives in ``oracle.c`` (plain C99, binary64 GEMM sums, binary32
quantization decisions); this module only builds that file with gcc and
marshals numpy arrays through ctypes.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")

FLAG_UE8M0 = 1
GROUP = 128
MX_GROUP = 32


def build(force: bool = False) -> str:
    """Compile oracle.c into liboracle.so with gcc (host code only)."""
    if force or not os.path.exists(_LIB) or os.path.getmtime(_LIB) < max(
        os.path.getmtime(_SRC), os.path.getmtime(os.path.join(_HERE, "oracle.h"))
    ):
        tmp = _LIB + ".tmp%d" % os.getpid()
        cmd = [
            "gcc", "-O2", "-std=c99", "-fPIC", "-shared", "-fopenmp",
            "-ffp-contract=off", "-fno-fast-math", "-Wall", "-Wextra",
            _SRC, "-o", tmp, "-lm",
        ]
        subprocess.run(cmd, check=True)
        os.replace(tmp, _LIB)
    return _LIB


_lib = None


def lib():
    global _lib
    if _lib is None:
        build()
        L = ctypes.CDLL(_LIB)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        U32 = ctypes.c_uint32
        L.oracle_e4m3_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e4m3_decode.restype = ctypes.c_double
        L.oracle_e4m3_encode.argtypes = [ctypes.c_float]
        L.oracle_e4m3_encode.restype = ctypes.c_uint8
        L.oracle_e4m3_encode_array.argtypes = [P, I64, P]
        L.oracle_e4m3_encode_array.restype = None
        L.oracle_scale_from_amax.argtypes = [ctypes.c_float, U32]
        L.oracle_scale_from_amax.restype = ctypes.c_float
        L.oracle_quant_1x128.argtypes = [P, I64, I64, U32, P, P]
        L.oracle_quant_128x128.argtypes = [P, I64, I64, U32, P, P]
        L.oracle_gemm_nt.argtypes = [P, P, P, P, I64, I64, I64, U32, P]
        L.oracle_gemm_nt_elems.argtypes = [P, P, P, P, I64, I64, I64, U32, P, P, I64, P]
        L.oracle_grouped_contiguous.argtypes = [P, P, P, P, P, I64, I64, I64,
                                                ctypes.c_int32, U32, P, P]
        L.oracle_contiguous_layout_violations.argtypes = [P, I64, ctypes.c_int32]
        L.oracle_contiguous_layout_violations.restype = I64
        L.oracle_grouped_masked.argtypes = [P, P, P, P, P, ctypes.c_int32, I64,
                                            I64, I64, U32, P, P]
        L.oracle_quant_mx.argtypes = [P, I64, I64, P, P]
        L.oracle_gemm_mx.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_gemm_mx_elems.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P]
        L.oracle_e2m1_decode.argtypes = [ctypes.c_uint8]
        L.oracle_e2m1_decode.restype = ctypes.c_double
        L.oracle_e2m1_encode.argtypes = [ctypes.c_float]
        L.oracle_e2m1_encode.restype = ctypes.c_uint8
        L.oracle_quant_mxfp4.argtypes = [P, I64, I64, P, P]
        L.oracle_gemm_mx_w4.argtypes = [P, P, P, P, I64, I64, I64, P]
        L.oracle_gemm_mx_w4_elems.argtypes = [P, P, P, P, I64, I64, I64, P, P, I64, P]
        L.oracle_num_threads.restype = ctypes.c_int
        L.oracle_set_num_threads.argtypes = [ctypes.c_int]
        L.oracle_set_num_threads.restype = None
        for fn in ("oracle_quant_1x128", "oracle_quant_128x128", "oracle_gemm_nt",
                   "oracle_gemm_nt_elems", "oracle_grouped_contiguous",
                   "oracle_grouped_masked", "oracle_quant_mx", "oracle_gemm_mx",
                   "oracle_gemm_mx_elems", "oracle_quant_mxfp4", "oracle_gemm_mx_w4",
                   "oracle_gemm_mx_w4_elems"):
            getattr(L, fn).restype = ctypes.c_int
        _lib = L
    return _lib


def _p(a: np.ndarray):
    assert a.flags["C_CONTIGUOUS"], "oracle arrays must be C-contiguous"
    return a.ctypes.data_as(ctypes.c_void_p)


def _check(rc: int, what: str):
    if rc != 0:
        raise ValueError(f"oracle {what}: bad arguments (rc={rc})")


def num_threads() -> int:
    return int(lib().oracle_num_threads())


def set_num_threads(n: int) -> None:
    """Threads used by the following calls; results do not depend on it."""
    lib().oracle_set_num_threads(int(n))


def e4m3_decode(codes) -> np.ndarray:
    """Decode uint8 codes to float64 values (NaN for the NaN codes)."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().oracle_e4m3_decode(c) for c in range(256)])
    return table[codes]


def e4m3_encode(values) -> np.ndarray:
    v = np.ascontiguousarray(values, dtype=np.float32)
    out = np.empty(v.shape, dtype=np.uint8)
    lib().oracle_e4m3_encode_array(_p(v), v.size, _p(out))
    return out


def scale_from_amax(amax: float, flags: int = 0) -> np.float32:
    return np.float32(lib().oracle_scale_from_amax(float(amax), flags))


def quant_1x128(x: np.ndarray, flags: int = 0):
    """x fp32 (M, K) -> (xq uint8 (M, K), sa fp32 (K/128, M))."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    M, K = x.shape
    xq = np.empty((M, K), np.uint8)
    sa = np.empty((K // GROUP, M), np.float32)
    _check(lib().oracle_quant_1x128(_p(x), M, K, flags, _p(xq), _p(sa)), "quant_1x128")
    return xq, sa


def quant_128x128(w: np.ndarray, flags: int = 0):
    """w fp32 (N, K) -> (wq uint8 (N, K), sb fp32 (ceil(N/128), K/128))."""
    w = np.ascontiguousarray(w, dtype=np.float32)
    N, K = w.shape
    wq = np.empty((N, K), np.uint8)
    sb = np.empty(((N + GROUP - 1) // GROUP, K // GROUP), np.float32)
    _check(lib().oracle_quant_128x128(_p(w), N, K, flags, _p(wq), _p(sb)), "quant_128x128")
    return wq, sb


def gemm_nt(xq, sa, wq, sb, flags: int = 0) -> np.ndarray:
    """Y (M, N) float64 = block-scaled X * W^T."""
    xq, sa, wq, sb = (np.ascontiguousarray(a) for a in (xq, sa, wq, sb))
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    _check(lib().oracle_gemm_nt(_p(xq), _p(sa), _p(wq), _p(sb), M, N, K, flags, _p(y)),
           "gemm_nt")
    return y


def gemm_nt_elems(xq, sa, wq, sb, m_idx, n_idx, flags: int = 0) -> np.ndarray:
    """Y[m_idx[i], n_idx[i]] for each i, float64."""
    xq, sa, wq, sb = (np.ascontiguousarray(a) for a in (xq, sa, wq, sb))
    M, K = xq.shape
    N = wq.shape[0]
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    y = np.empty(m_idx.shape, np.float64)
    _check(lib().oracle_gemm_nt_elems(_p(xq), _p(sa), _p(wq), _p(sb), M, N, K, flags,
                                      _p(m_idx), _p(n_idx), m_idx.size, _p(y)),
           "gemm_nt_elems")
    return y


def grouped_contiguous(xq, sa, wq, sb, m_indices, E: int, flags: int = 0):
    """Returns (y float64 (M, N), written bool (M,)).  wq is (E*N, K) or (E, N, K)."""
    xq, sa = np.ascontiguousarray(xq), np.ascontiguousarray(sa)
    M, K = xq.shape
    wq = np.ascontiguousarray(wq).reshape(-1, K)
    N = wq.shape[0] // E if E else 0
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    idx = np.ascontiguousarray(m_indices, dtype=np.int32)
    y = np.zeros((M, N), np.float64)
    written = np.zeros(M, np.uint8)
    _check(lib().oracle_grouped_contiguous(_p(xq), _p(sa), _p(wq), _p(sb), _p(idx), M, N, K,
                                           E, flags, _p(y), _p(written)),
           "grouped_contiguous")
    return y, written.astype(bool)


def contiguous_layout_violations(m_indices, E: int) -> int:
    idx = np.ascontiguousarray(m_indices, dtype=np.int32)
    return int(lib().oracle_contiguous_layout_violations(_p(idx), idx.size, E))


def grouped_masked(xq, sa, wq, sb, masked_m, E: int, max_m: int, flags: int = 0):
    """xq (E*max_m, K), sa (K/128, E*max_m), wq (E*N, K), sb (E*N/128, K/128).

    Returns (y float64 (E*max_m, N), written bool (E*max_m,))."""
    xq, sa = np.ascontiguousarray(xq), np.ascontiguousarray(sa)
    MT, K = xq.shape
    wq = np.ascontiguousarray(wq).reshape(-1, K)
    N = wq.shape[0] // E if E else 0
    sb = np.ascontiguousarray(sb, dtype=np.float32)
    mm = np.ascontiguousarray(masked_m, dtype=np.int32)
    y = np.zeros((MT, N), np.float64)
    written = np.zeros(MT, np.uint8)
    _check(lib().oracle_grouped_masked(_p(xq), _p(sa), _p(wq), _p(sb), _p(mm), E, max_m, N, K,
                                       flags, _p(y), _p(written)),
           "grouped_masked")
    return y, written.astype(bool)


def quant_mx(x: np.ndarray):
    """MXFP8: x fp32 (R, K) -> (q uint8 (R, K), e uint8 (R, K/32)); 2^(e-127) is
    the scale of each 1x32 group."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    q = np.empty((R, K), np.uint8)
    e = np.empty((R, K // MX_GROUP), np.uint8)
    _check(lib().oracle_quant_mx(_p(x), R, K, _p(q), _p(e)), "quant_mx")
    return q, e


def gemm_mx(xq, ea, wq, eb) -> np.ndarray:
    """Y (M, N) float64 = MX-scaled X * W^T."""
    xq, ea, wq, eb = (np.ascontiguousarray(a, dtype=np.uint8) for a in (xq, ea, wq, eb))
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    _check(lib().oracle_gemm_mx(_p(xq), _p(ea), _p(wq), _p(eb), M, N, K, _p(y)), "gemm_mx")
    return y


def gemm_mx_elems(xq, ea, wq, eb, m_idx, n_idx) -> np.ndarray:
    """Y[m_idx[i], n_idx[i]] of the MX GEMM, float64."""
    xq, ea, wq, eb = (np.ascontiguousarray(a, dtype=np.uint8) for a in (xq, ea, wq, eb))
    M, K = xq.shape
    N = wq.shape[0]
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    y = np.empty(m_idx.shape, np.float64)
    _check(lib().oracle_gemm_mx_elems(_p(xq), _p(ea), _p(wq), _p(eb), M, N, K, _p(m_idx),
                                      _p(n_idx), m_idx.size, _p(y)), "gemm_mx_elems")
    return y


def e2m1_decode(codes) -> np.ndarray:
    """Decode E2M1 nibbles (0..15) to float64 values."""
    codes = np.asarray(codes, dtype=np.uint8)
    table = np.array([lib().oracle_e2m1_decode(c) for c in range(16)])
    return table[codes & 0xF]


def e2m1_encode(values) -> np.ndarray:
    v = np.asarray(values, dtype=np.float32)
    return np.array([lib().oracle_e2m1_encode(float(t)) for t in v.ravel()], np.uint8).reshape(v.shape)


def quant_mxfp4(x: np.ndarray):
    """MXFP4: x fp32 (R, K) -> (q uint8 (R, K/2) packed nibbles, element k in
    byte k/2 (low nibble for even k); e uint8 (R, K/32))."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    R, K = x.shape
    q = np.empty((R, K // 2), np.uint8)
    e = np.empty((R, K // MX_GROUP), np.uint8)
    _check(lib().oracle_quant_mxfp4(_p(x), R, K, _p(q), _p(e)), "quant_mxfp4")
    return q, e


def gemm_mx_w4(xq, ea, wq, eb) -> np.ndarray:
    """Y (M, N) float64 = MXFP8 X * (MXFP4 W)^T."""
    xq, ea, wq, eb = (np.ascontiguousarray(a, dtype=np.uint8) for a in (xq, ea, wq, eb))
    M, K = xq.shape
    N = wq.shape[0]
    y = np.empty((M, N), np.float64)
    _check(lib().oracle_gemm_mx_w4(_p(xq), _p(ea), _p(wq), _p(eb), M, N, K, _p(y)), "gemm_mx_w4")
    return y


def gemm_mx_w4_elems(xq, ea, wq, eb, m_idx, n_idx) -> np.ndarray:
    xq, ea, wq, eb = (np.ascontiguousarray(a, dtype=np.uint8) for a in (xq, ea, wq, eb))
    M, K = xq.shape
    N = wq.shape[0]
    m_idx = np.ascontiguousarray(m_idx, dtype=np.int64)
    n_idx = np.ascontiguousarray(n_idx, dtype=np.int64)
    y = np.empty(m_idx.shape, np.float64)
    _check(lib().oracle_gemm_mx_w4_elems(_p(xq), _p(ea), _p(wq), _p(eb), M, N, K, _p(m_idx),
                                         _p(n_idx), m_idx.size, _p(y)), "gemm_mx_w4_elems")
    return y
