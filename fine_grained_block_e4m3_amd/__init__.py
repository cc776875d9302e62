"""Fine-grained block-scaled E4M3 GEMM for AMD MI355X (gfx950).

Thin ctypes binding over ``libfp8gemm.so`` (C ABI in ``include/fp8gemm.h``).
Every function below only checks tensor shapes/dtypes/devices, allocates the
outputs through torch and passes raw device pointers plus the current HIP
stream to the library; all arithmetic runs in the library's HIP kernels.  If
the library is not built, or no GPU is visible, calls raise -- there is no
CPU fallback.

Names follow the C ABI: ``quant_1x128``, ``quant_128x128``, ``gemm_nt``,
``grouped_gemm_contiguous``, ``grouped_gemm_masked``,
``get_mk_alignment_for_contiguous_layout``.
"""
from __future__ import annotations

import ctypes
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_HERE, "libfp8gemm.so")

FLAG_UE8M0 = 1
FLAG_FAST_ACCUM = 2
PLAN_MX = 0x100
PLAN_QOUT = 0x200
LAYOUT = {"dense": 0, "contiguous": 1, "masked": 2}

STATUS = {
    0: "FP8_OK",
    1: "FP8_ERR_INVALID_ARG",
    2: "FP8_ERR_SHAPE",
    3: "FP8_ERR_ALIGNMENT",
    4: "FP8_ERR_UNSUPPORTED",
    5: "FP8_ERR_NO_DEVICE",
    6: "FP8_ERR_LAUNCH",
    7: "FP8_ERR_SCRATCH",
}

# Exported C symbols (kept in step with include/fp8gemm.h by the tests).
SYMBOLS = (
    "fp8_quant_1x128",
    "fp8_quant_128x128",
    "fp8_gemm_nt",
    "fp8_gemm_nt_ws",
    "fp8_gemm_nt_noalloc",
    "fp8_gemm_workspace_size",
    "fp8_gemm_plan",
    "fp8_gemm_nt_qout",
    "fp8_grouped_gemm_contiguous",
    "fp8_grouped_gemm_masked",
    "fp8_quant_mx",
    "fp8_gemm_nt_mx",
    "fp8_quant_mxfp4",
    "fp8_gemm_nt_mx_w4",
    "fp8_get_mk_alignment_for_contiguous_layout",
    "fp8_status_string",
)


class GemmPlan(ctypes.Structure):
    """fp8_gemm_plan_t: the kernel instances a GEMM call launches."""
    _fields_ = [("exact", ctypes.c_int32), ("kernel", ctypes.c_int32), ("tile_m", ctypes.c_int32),
                ("tile_n", ctypes.c_int32), ("waves", ctypes.c_int32), ("grid", ctypes.c_int32),
                ("tiles", ctypes.c_int64), ("main_rows", ctypes.c_int64), ("tail_tile_m", ctypes.c_int32),
                ("tail_tile_n", ctypes.c_int32), ("tail_tiles", ctypes.c_int64), ("k_splits", ctypes.c_int32),
                ("workspace_bytes", ctypes.c_size_t), ("main_cols", ctypes.c_int64),
                ("paired", ctypes.c_int32), ("mid_tile_m", ctypes.c_int32), ("mid_tile_n", ctypes.c_int32),
                ("mid_tiles", ctypes.c_int64)]

    def as_dict(self) -> dict:
        return {name: getattr(self, name) for name, _ in self._fields_}


class Fp8GemmError(RuntimeError):
    def __init__(self, fn: str, status: int, msg: str):
        super().__init__(f"{fn}: {STATUS.get(status, status)} ({msg})")
        self.status = status


_lib = None


def load_library(path: str = LIB_PATH) -> ctypes.CDLL:
    """Load libfp8gemm.so (no GPU needed to load it).  Raises if absent."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(path):
        raise ImportError(
            f"{path} is not built; run `python -m fine_grained_block_e4m3_amd.build` "
            "(hipcc, gfx950). There is no CPU fallback.")
    L = ctypes.CDLL(path)
    P, I64, I32, U32 = ctypes.c_void_p, ctypes.c_int64, ctypes.c_int32, ctypes.c_uint32
    L.fp8_quant_1x128.argtypes = [P, I64, I64, P, P, U32, P]
    L.fp8_quant_128x128.argtypes = [P, I64, I64, P, P, U32, P]
    L.fp8_gemm_nt.argtypes = [P, P, P, P, P, I64, I64, I64, U32, P]
    L.fp8_gemm_nt_ws.argtypes = [P, P, P, P, P, I64, I64, I64, U32, P, ctypes.c_size_t, P]
    L.fp8_gemm_nt_noalloc.argtypes = [P, P, P, P, P, I64, I64, I64, U32, P]
    L.fp8_gemm_workspace_size.argtypes = [I64, I64, I64, U32]
    L.fp8_gemm_workspace_size.restype = ctypes.c_size_t
    L.fp8_gemm_plan.argtypes = [I32, I64, I64, I64, U32, I32, ctypes.c_size_t, ctypes.POINTER(GemmPlan)]
    L.fp8_gemm_nt_qout.argtypes = [P, P, P, P, P, P, I64, I64, I64, U32, P]
    L.fp8_grouped_gemm_contiguous.argtypes = [P, P, P, P, P, P, I64, I64, I64, I32, U32, P]
    L.fp8_grouped_gemm_masked.argtypes = [P, P, P, P, P, P, I32, I64, I64, I64, U32, P]
    L.fp8_quant_mx.argtypes = [P, I64, I64, P, P, P]
    L.fp8_gemm_nt_mx.argtypes = [P, P, P, P, P, I64, I64, I64, U32, P]
    L.fp8_quant_mxfp4.argtypes = [P, I64, I64, P, P, P]
    L.fp8_gemm_nt_mx_w4.argtypes = [P, P, P, P, P, I64, I64, I64, U32, P]
    for fn in ("fp8_quant_1x128", "fp8_quant_128x128", "fp8_gemm_nt", "fp8_gemm_nt_ws", "fp8_gemm_nt_noalloc",
               "fp8_gemm_plan",
               "fp8_gemm_nt_qout",
               "fp8_grouped_gemm_contiguous", "fp8_grouped_gemm_masked", "fp8_quant_mx",
               "fp8_gemm_nt_mx", "fp8_quant_mxfp4", "fp8_gemm_nt_mx_w4"):
        getattr(L, fn).restype = ctypes.c_int
    L.fp8_get_mk_alignment_for_contiguous_layout.argtypes = []
    L.fp8_get_mk_alignment_for_contiguous_layout.restype = I32
    L.fp8_status_string.argtypes = [ctypes.c_int]
    L.fp8_status_string.restype = ctypes.c_char_p
    _lib = L
    return L


def _check(fn: str, status: int) -> None:
    if status != 0:
        msg = load_library().fp8_status_string(status).decode()
        raise Fp8GemmError(fn, status, msg)


def _stream(t: torch.Tensor):
    return ctypes.c_void_p(torch.cuda.current_stream(t.device).cuda_stream)


def _need(t: torch.Tensor, name: str, dtype: torch.dtype, ndim: int) -> None:
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor (no CPU path exists)")
    if t.dtype != dtype:
        raise TypeError(f"{name} must be {dtype}, got {t.dtype}")
    if t.dim() != ndim:
        raise ValueError(f"{name} must have {ndim} dims, got {tuple(t.shape)}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")


def _out(t, name: str, dtype: torch.dtype, shape, like: torch.Tensor) -> torch.Tensor:
    """A caller's output buffer: the kernels write exactly this shape, so any
    other shape, type, layout or device is refused before a launch."""
    _need(t, name, dtype, len(shape))
    if tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} must have shape {tuple(shape)}, got {tuple(t.shape)}")
    if t.device != like.device:
        raise ValueError(f"{name} is on {t.device}, the inputs on {like.device}")
    return t


def _same_device(*ts: torch.Tensor) -> None:
    d = ts[0].device
    for t in ts[1:]:
        if t.device != d:
            raise ValueError(f"operands on different devices: {d} and {t.device}")


def _ptr(t: torch.Tensor):
    return ctypes.c_void_p(t.data_ptr())


def _flags(ue8m0: bool, fast_accum: bool = False) -> int:
    return (FLAG_UE8M0 if ue8m0 else 0) | (FLAG_FAST_ACCUM if fast_accum else 0)


def gemm_plan(layout: str, M: int, N: int, K: int, ue8m0: bool = False, fast_accum: bool = False,
              mx: bool = False, qout: bool = False, compute_units: int = 256,
              workspace_bytes: int = 0) -> dict:
    """The kernel instances a GEMM call of this shape launches (host-side
    arithmetic only; no GPU needed).  layout: dense, contiguous or masked
    (max_m as M)."""
    L = load_library()
    flags = _flags(ue8m0, fast_accum) | (PLAN_MX if mx else 0) | (PLAN_QOUT if qout else 0)
    plan = GemmPlan()
    _check("fp8_gemm_plan", L.fp8_gemm_plan(LAYOUT[layout], M, N, K, flags, compute_units, workspace_bytes,
                                            ctypes.byref(plan)))
    return plan.as_dict()


def get_mk_alignment_for_contiguous_layout() -> int:
    return int(load_library().fp8_get_mk_alignment_for_contiguous_layout())


def quant_1x128(x: torch.Tensor, ue8m0: bool = False, out=None):
    """x fp32 (M, K) -> (xq uint8 (M, K), sa fp32 (K/128, M))."""
    L = load_library()
    _need(x, "x", torch.float32, 2)
    M, K = x.shape
    if out is None:
        xq = torch.empty((M, K), dtype=torch.uint8, device=x.device)
        sa = torch.empty((K // 128, M), dtype=torch.float32, device=x.device)
    else:
        xq = _out(out[0], "out[0]", torch.uint8, (M, K), x)
        sa = _out(out[1], "out[1]", torch.float32, (K // 128, M), x)
    _check("fp8_quant_1x128", L.fp8_quant_1x128(_ptr(x), M, K, _ptr(xq), _ptr(sa),
                                                _flags(ue8m0), _stream(x)))
    return xq, sa


def quant_128x128(w: torch.Tensor, ue8m0: bool = False, out=None):
    """w fp32 (N, K) -> (wq uint8 (N, K), sb fp32 (ceil(N/128), K/128))."""
    L = load_library()
    _need(w, "w", torch.float32, 2)
    N, K = w.shape
    if out is None:
        wq = torch.empty((N, K), dtype=torch.uint8, device=w.device)
        sb = torch.empty(((N + 127) // 128, K // 128), dtype=torch.float32, device=w.device)
    else:
        wq = _out(out[0], "out[0]", torch.uint8, (N, K), w)
        sb = _out(out[1], "out[1]", torch.float32, ((N + 127) // 128, K // 128), w)
    _check("fp8_quant_128x128", L.fp8_quant_128x128(_ptr(w), N, K, _ptr(wq), _ptr(sb),
                                                    _flags(ue8m0), _stream(w)))
    return wq, sb


def gemm_nt(xq, sa, wq, sb, ue8m0: bool = False, fast_accum: bool = False, out=None,
            workspace=None) -> torch.Tensor:
    """Y (M, N) bf16 = block-scaled X * W^T.  fast_accum: block partials from
    the FP8 matrix instruction (see FP8_FLAG_FAST_ACCUM).  With fast_accum and
    a decode-sized M the library splits K when given a workspace: a uint8
    device tensor of at least fp8_gemm_workspace_size() bytes, allocated here
    through torch when not passed."""
    L = load_library()
    _need(xq, "xq", torch.uint8, 2)
    _need(wq, "wq", torch.uint8, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or sa.shape != (K // 128, M) or sb.shape != ((N + 127) // 128, K // 128):
        raise ValueError("gemm_nt: inconsistent operand shapes")
    _same_device(xq, sa, wq, sb)
    y = _out(out, "out", torch.bfloat16, (M, N), xq) if out is not None \
        else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    flags = _flags(ue8m0, fast_accum)
    if workspace is None and M and N and K:
        nbytes = int(L.fp8_gemm_workspace_size(M, N, K, flags))
        if nbytes:
            workspace = torch.empty(nbytes, dtype=torch.uint8, device=xq.device)
    if workspace is not None:
        _need(workspace, "workspace", torch.uint8, 1)
        _same_device(xq, workspace)
        ws, ws_bytes = _ptr(workspace), workspace.numel()
    else:
        ws, ws_bytes = None, 0
    _check("fp8_gemm_nt_ws", L.fp8_gemm_nt_ws(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sb), _ptr(y),
                                              M, N, K, flags, ws, ws_bytes, _stream(xq)))
    return y


def gemm_nt_qout(xq, sa, wq, sb, ue8m0: bool = False, fast_accum: bool = False, out=None):
    """Block-scaled X * W^T written quantized for the next GEMM: (yq uint8
    (M, N) E4M3 codes, sy fp32 (N/128, M) 1x128 scales); N % 128 == 0."""
    L = load_library()
    _need(xq, "xq", torch.uint8, 2)
    _need(wq, "wq", torch.uint8, 2)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or sa.shape != (K // 128, M) or sb.shape != ((N + 127) // 128, K // 128):
        raise ValueError("gemm_nt_qout: inconsistent operand shapes")
    _same_device(xq, sa, wq, sb)
    if out is None:
        yq = torch.empty((M, N), dtype=torch.uint8, device=xq.device)
        sy = torch.empty((N // 128, M), dtype=torch.float32, device=xq.device)
    else:
        yq = _out(out[0], "out[0]", torch.uint8, (M, N), xq)
        sy = _out(out[1], "out[1]", torch.float32, (N // 128, M), xq)
    _check("fp8_gemm_nt_qout", L.fp8_gemm_nt_qout(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sb), _ptr(yq),
                                                  _ptr(sy), M, N, K, _flags(ue8m0, fast_accum),
                                                  _stream(xq)))
    return yq, sy


def grouped_gemm_contiguous(xq, sa, wq, sb, m_indices, ue8m0: bool = False, fast_accum: bool = False,
                            out=None) -> torch.Tensor:
    """xq (M, K), sa (K/128, M), wq (E, N, K), sb (E, N/128, K/128), m_indices int32 (M)."""
    L = load_library()
    _need(xq, "xq", torch.uint8, 2)
    _need(wq, "wq", torch.uint8, 3)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 3)
    _need(m_indices, "m_indices", torch.int32, 1)
    M, K = xq.shape
    E, N, _ = wq.shape
    if wq.shape[2] != K or sa.shape != (K // 128, M) or sb.shape != (E, N // 128, K // 128) \
            or m_indices.shape[0] != M:
        raise ValueError("grouped_gemm_contiguous: inconsistent operand shapes")
    _same_device(xq, sa, wq, sb, m_indices)
    y = _out(out, "out", torch.bfloat16, (M, N), xq) if out is not None \
        else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check("fp8_grouped_gemm_contiguous",
           L.fp8_grouped_gemm_contiguous(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sb), _ptr(m_indices),
                                         _ptr(y), M, N, K, E, _flags(ue8m0, fast_accum), _stream(xq)))
    return y


def grouped_gemm_masked(xq, sa, wq, sb, masked_m, ue8m0: bool = False, fast_accum: bool = False,
                        out=None) -> torch.Tensor:
    """xq (E, max_m, K), sa (K/128, E*max_m), wq (E, N, K), sb (E, N/128, K/128),
    masked_m int32 (E).  Returns y (E, max_m, N) bf16 (rows past masked_m untouched)."""
    L = load_library()
    _need(xq, "xq", torch.uint8, 3)
    _need(wq, "wq", torch.uint8, 3)
    _need(sa, "sa", torch.float32, 2)
    _need(sb, "sb", torch.float32, 3)
    _need(masked_m, "masked_m", torch.int32, 1)
    E, max_m, K = xq.shape
    N = wq.shape[1]
    if wq.shape != (E, N, K) or sa.shape != (K // 128, E * max_m) \
            or sb.shape != (E, N // 128, K // 128) or masked_m.shape[0] != E:
        raise ValueError("grouped_gemm_masked: inconsistent operand shapes")
    _same_device(xq, sa, wq, sb, masked_m)
    y = _out(out, "out", torch.bfloat16, (E, max_m, N), xq) if out is not None \
        else torch.empty((E, max_m, N), dtype=torch.bfloat16, device=xq.device)
    _check("fp8_grouped_gemm_masked",
           L.fp8_grouped_gemm_masked(_ptr(xq), _ptr(sa), _ptr(wq), _ptr(sb), _ptr(masked_m),
                                     _ptr(y), E, max_m, N, K, _flags(ue8m0, fast_accum), _stream(xq)))
    return y


def quant_mx(x: torch.Tensor, out=None):
    """MXFP8: x fp32 (R, K) -> (q uint8 (R, K), e int32 (K/128, R)).  e holds the
    packed scale bytes: byte t of e[kb, r] is the exponent byte b of 1x32 group
    4*kb + t of row r, whose scale is 2^(b - 127)."""
    L = load_library()
    _need(x, "x", torch.float32, 2)
    R, K = x.shape
    if out is None:
        q = torch.empty((R, K), dtype=torch.uint8, device=x.device)
        e = torch.empty((K // 128, R), dtype=torch.int32, device=x.device)
    else:
        q = _out(out[0], "out[0]", torch.uint8, (R, K), x)
        e = _out(out[1], "out[1]", torch.int32, (K // 128, R), x)
    _check("fp8_quant_mx", L.fp8_quant_mx(_ptr(x), R, K, _ptr(q), _ptr(e), _stream(x)))
    return q, e


def gemm_nt_mx(xq, ea, wq, eb, out=None) -> torch.Tensor:
    """Y (M, N) bf16 = MXFP8 X * W^T; ea (K/128, M) and eb (K/128, N) are the
    packed scale tables that quant_mx writes."""
    L = load_library()
    _need(xq, "xq", torch.uint8, 2)
    _need(wq, "wq", torch.uint8, 2)
    _need(ea, "ea", torch.int32, 2)
    _need(eb, "eb", torch.int32, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] != K or ea.shape != (K // 128, M) or eb.shape != (K // 128, N):
        raise ValueError("gemm_nt_mx: inconsistent operand shapes")
    _same_device(xq, ea, wq, eb)
    y = _out(out, "out", torch.bfloat16, (M, N), xq) if out is not None \
        else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check("fp8_gemm_nt_mx", L.fp8_gemm_nt_mx(_ptr(xq), _ptr(ea), _ptr(wq), _ptr(eb), _ptr(y),
                                              M, N, K, 0, _stream(xq)))
    return y


def quant_mxfp4(w: torch.Tensor, out=None):
    """MXFP4 weights: w fp32 (R, K) -> (q uint8 (R, K/2), two E2M1 nibbles per
    byte, the even element low; e int32 (K/128, R) packed scale bytes)."""
    L = load_library()
    _need(w, "w", torch.float32, 2)
    R, K = w.shape
    if out is None:
        q = torch.empty((R, K // 2), dtype=torch.uint8, device=w.device)
        e = torch.empty((K // 128, R), dtype=torch.int32, device=w.device)
    else:
        q = _out(out[0], "out[0]", torch.uint8, (R, K // 2), w)
        e = _out(out[1], "out[1]", torch.int32, (K // 128, R), w)
    _check("fp8_quant_mxfp4", L.fp8_quant_mxfp4(_ptr(w), R, K, _ptr(q), _ptr(e), _stream(w)))
    return q, e


def gemm_nt_mx_w4(xq, ea, wq, eb, out=None) -> torch.Tensor:
    """Y (M, N) bf16 = MXFP8 X * (MXFP4 W)^T; wq (N, K/2) packed nibbles."""
    L = load_library()
    _need(xq, "xq", torch.uint8, 2)
    _need(wq, "wq", torch.uint8, 2)
    _need(ea, "ea", torch.int32, 2)
    _need(eb, "eb", torch.int32, 2)
    M, K = xq.shape
    N = wq.shape[0]
    if wq.shape[1] * 2 != K or ea.shape != (K // 128, M) or eb.shape != (K // 128, N):
        raise ValueError("gemm_nt_mx_w4: inconsistent operand shapes")
    _same_device(xq, ea, wq, eb)
    y = _out(out, "out", torch.bfloat16, (M, N), xq) if out is not None \
        else torch.empty((M, N), dtype=torch.bfloat16, device=xq.device)
    _check("fp8_gemm_nt_mx_w4", L.fp8_gemm_nt_mx_w4(_ptr(xq), _ptr(ea), _ptr(wq), _ptr(eb), _ptr(y),
                                                    M, N, K, 0, _stream(xq)))
    return y
