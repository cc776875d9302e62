"""Helpers shared by the GPU parity tests (not a test module)."""
from __future__ import annotations

import sys

import numpy as np
import torch

# |y - ref| <= REL * |ref| + ABS_RMS * rms(ref), rms over the compared elements
REL = 8e-3
ABS_RMS = 1e-3
SENTINEL = 0x7FA5          # a BF16 NaN bit pattern no kernel ever produces


def say(*a) -> None:
    """Name the case on stdout before each GPU step (flushed)."""
    print(*a, flush=True)
    sys.stdout.flush()


def dev(a: np.ndarray) -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a)).cuda()


def host(t: torch.Tensor) -> np.ndarray:
    torch.cuda.synchronize()
    return t.cpu().numpy()


def bf16_bits(t: torch.Tensor) -> np.ndarray:
    return host(t.view(torch.int16)).view(np.uint16)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def sentinel_like(shape, device="cuda") -> torch.Tensor:
    t = torch.empty(shape, dtype=torch.int16, device=device)
    t.fill_(SENTINEL)            # 0x7FA5 < 2^15: the same bits as int16
    return t.view(torch.bfloat16)


def guarded(shape, guard: int = 2048):
    """A BF16 output with `guard` sentinel elements before and after it.
    Returns (full buffer, view of the output)."""
    n = int(np.prod(shape))
    full = sentinel_like((n + 2 * guard + 8,))
    # keep the output 16-byte aligned: guard is a multiple of 8 elements
    out = full[guard:guard + n].view(*shape)
    return full, out


def check_guards(full: torch.Tensor, n: int, guard: int = 2048) -> None:
    bits = bf16_bits(full)
    assert np.all(bits[:guard] == SENTINEL), "write before the output"
    assert np.all(bits[guard + n:] == SENTINEL), "write after the output"


def assert_close(y_bits: np.ndarray, ref: np.ndarray, what: str = "") -> dict:
    """Element-wise tolerance check; returns error statistics."""
    y = bf16_to_f64(np.asarray(y_bits))
    ref = np.asarray(ref, dtype=np.float64)
    assert y.shape == ref.shape, (y.shape, ref.shape)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    if ref.size == 0:
        return {"n": 0}
    rms = float(np.sqrt(np.mean(ref * ref)))
    err = np.abs(y - ref)
    bound = REL * np.abs(ref) + ABS_RMS * rms
    bad = err > bound
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())}/{bad.size} elements outside tolerance; first "
            f"{[(tuple(i), float(y[tuple(i)]), float(ref[tuple(i)])) for i in idx]}")
    return {"n": int(ref.size), "max_rel": float(np.max(err / np.maximum(np.abs(ref), 1e-30))),
            "max_abs_over_rms": float(np.max(err) / max(rms, 1e-30))}


def _dec_table() -> np.ndarray:
    import oracle
    return oracle.e4m3_decode(np.arange(256))


def fp8_mfma_error_bound(xq, sa, wq, sb, ref, pow2: bool = False) -> np.ndarray:
    """Per-element bound on |y - ref| for the FP8-MFMA accumulation path.

    Measured model of the gfx950 FP8 matrix instruction: within each group of 8
    consecutive K positions every product is truncated toward zero to a
    multiple of 2^(E-13), where 2^E <= the group's largest |product|; the group
    sums then combine in FP32.  A group therefore loses less than
    8 * 2^-13 * max|p| = 2^-10 * max|p| <= 2^-10 * max|a| * max|b|.  Summed over
    groups with their block scales this is a (group-max) matrix product.  Add
    BF16 output rounding (2^-9 |y|) and FP32 promotion/accumulation rounding.
    With pow2 (scaled instruction, K accumulated in its FP32 accumulator) the
    running sum is rounded once per 128-K block as well (absorbed in the
    2^-16 term)."""
    DEC = _dec_table()
    M, K = xq.shape
    N = wq.shape[0]
    G = K // 8
    sa64 = sa.astype(np.float64)
    sb64 = sb.astype(np.float64)
    if pow2:
        with np.errstate(divide="ignore"):          # a zero scale stays zero
            sa64 = np.exp2(np.floor(np.log2(sa64)))
            sb64 = np.exp2(np.floor(np.log2(sb64)))
    sa_g = np.repeat(sa64.T, 16, axis=1)                                   # (M, G)
    sb_g = np.repeat(np.repeat(sb64, 128, axis=0)[:N], 16, axis=1)         # (N, G)
    amax = np.abs(DEC[xq]).reshape(M, G, 8).max(axis=2) * sa_g
    bmax = np.abs(DEC[wq]).reshape(N, G, 8).max(axis=2) * sb_g
    trunc = 2.0 ** -10 * (amax @ bmax.T)
    sx = np.repeat(sa64.T, 128, axis=1)
    sw = np.repeat(np.repeat(sb64, 128, axis=0)[:N], 128, axis=1)
    absprod = (np.abs(DEC[xq]) * sx) @ (np.abs(DEC[wq]) * sw).T
    return 2.0 ** -8 * np.abs(ref) + 1.01 * trunc + 2.0 ** -16 * absprod


def assert_close_or_bounded(y_bits, ref, bound, what: str = "", max_beyond_frac: float = 1e-4) -> dict:
    """For the opt-in FP8-instruction path (FP8_FLAG_FAST_ACCUM, MX): every
    element within the benchmark spec's tolerance or within `bound`, the bound of
    the measured FP8-MFMA truncation model; and the elements outside the
    tolerance (reported as beyond_strict) at most max_beyond_frac of them,
    rounded up, so that a regression that moves many elements past the
    tolerance fails even while they stay inside the model's bound."""
    y = bf16_to_f64(np.asarray(y_bits))
    ref = np.asarray(ref, dtype=np.float64)
    assert np.all(np.isfinite(y)), f"{what}: non-finite output"
    rms = float(np.sqrt(np.mean(ref * ref))) if ref.size else 0.0
    err = np.abs(y - ref)
    strict = REL * np.abs(ref) + ABS_RMS * rms
    bad = (err > strict) & (err > bound)
    if np.any(bad):
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} elements beyond both the tolerance and the "
                             f"FP8-MFMA model bound; first "
                             f"{[(tuple(i), float(y[tuple(i)]), float(ref[tuple(i)]), float(bound[tuple(i)])) for i in idx]}")
    beyond = int(np.sum(err > strict))
    ceiling = int(np.ceil(max_beyond_frac * ref.size))
    assert beyond <= ceiling, (f"{what}: {beyond} of {ref.size} elements outside the tolerance "
                               f"(ceiling {ceiling})")
    return {"n": int(ref.size), "beyond_strict": beyond, "ceiling": ceiling}
