"""Seeded synthetic inputs for the block-scaled E4M3 GEMM workloads.

This module only draws random numbers: it holds none of the method's
arithmetic (no scales, no quantization, no products).  Both the GPU path's
tests/benchmark and the CPU oracle are fed from it.

Workload shapes follow the DeepSeek-V3-like shapes used with the DeepGEMM
kernel (K = 7168 is that model's hidden size, per the DeepGEMM page, section
"细粒度缩放在 GEMM 层面引爆的两个问题").  No public dataset is involved: every
tensor is drawn from numpy's PCG64 generator with a fixed seed.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

GROUP = 128


@dataclass
class Workload:
    kind: str                 # "dense" | "contiguous" | "masked"
    name: str
    x: np.ndarray             # fp32 activations (M, K); grouped: (M_total, K)
    w: np.ndarray             # fp32 weights (N, K); grouped: (E*N, K)
    M: int
    N: int
    K: int
    E: int = 1
    max_m: int = 0
    ue8m0: bool = False
    m_indices: np.ndarray | None = None   # contiguous: int32 per row, -1 = padding
    masked_m: np.ndarray | None = None    # masked: int32 per expert
    meta: dict = field(default_factory=dict)


def _outliers(rng: np.random.Generator, a: np.ndarray, frac: float, mult: float) -> None:
    """Multiply exactly round(frac * a.size) distinct entries by `mult` in place."""
    if frac <= 0:
        return
    n = int(round(frac * a.size))
    idx = rng.choice(a.size, n, replace=False)
    flat = a.reshape(-1)
    flat[idx] *= np.float32(mult)


def dense(M: int, N: int, K: int, seed: int, outlier_frac: float = 0.0,
          outlier_mult: float = 1.0, w_std: float = 1.0, name: str = "dense") -> Workload:
    """X ~ N(0,1) (M,K), W ~ N(0, w_std^2) (N,K), then outliers, X first."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal((M, K), dtype=np.float32)
    _outliers(rng, x, outlier_frac, outlier_mult)
    w = rng.standard_normal((N, K), dtype=np.float32)
    if w_std != 1.0:
        w *= np.float32(w_std)
    _outliers(rng, w, outlier_frac, outlier_mult)
    return Workload("dense", name, x, w, M, N, K)


def contiguous(E: int, tokens: int, N: int, K: int, seed: int, name: str = "contiguous",
               counts: np.ndarray | None = None) -> Workload:
    """MoE prefill routing: p ~ Dirichlet(1^E), counts ~ Multinomial(tokens, p).

    Expert e's rows are one segment padded up to a multiple of 128 rows; the
    segments follow each other in expert order.  m_indices is e on the valid
    rows and -1 on the padding rows, whose X is zero.  X, W ~ N(0,1).
    """
    rng = np.random.default_rng(seed)
    if counts is None:
        p = rng.dirichlet(np.ones(E))
        counts = rng.multinomial(tokens, p)
    counts = np.asarray(counts, dtype=np.int64)
    padded = ((counts + GROUP - 1) // GROUP) * GROUP
    M = int(padded.sum())
    m_indices = np.full(M, -1, np.int32)
    off = 0
    for e in range(E):
        m_indices[off:off + counts[e]] = e
        off += int(padded[e])
    x = np.zeros((M, K), np.float32)
    valid = m_indices >= 0
    x[valid] = rng.standard_normal((int(valid.sum()), K), dtype=np.float32)
    w = rng.standard_normal((E * N, K), dtype=np.float32)
    return Workload("contiguous", name, x, w, M, N, K, E=E, m_indices=m_indices,
                    meta={"counts": counts.tolist(), "tokens": int(counts.sum())})


def masked(E: int, max_m: int, N: int, K: int, seed: int, ue8m0: bool = True,
           name: str = "masked", masked_m: np.ndarray | None = None) -> Workload:
    """MoE decode buffers: valid_m[e] ~ U{0..max_m}; X (E*max_m, K) and W (E*N, K)
    ~ N(0,1); rows past valid_m hold N(0,1) garbage that must not be read."""
    rng = np.random.default_rng(seed)
    if masked_m is None:
        masked_m = rng.integers(0, max_m + 1, size=E)
    masked_m = np.asarray(masked_m, dtype=np.int32)
    x = rng.standard_normal((E * max_m, K), dtype=np.float32)
    w = rng.standard_normal((E * N, K), dtype=np.float32)
    return Workload("masked", name, x, w, E * max_m, N, K, E=E, max_m=max_m, ue8m0=ue8m0,
                    masked_m=masked_m)


# The five headline workloads.  Seed = configuration number.
CONFIG_NAMES = {
    1: "dense M=128 N=256 K=512, 1% outliers x50",
    2: "dense prefill M=4096 N=7168 K=7168, 0.1% outliers x100",
    3: "dense decode M=64 N=24576 K=1536, W ~ N(0, 0.02^2)",
    4: "contiguous MoE E=8 tokens=8192 N=4096 K=7168",
    5: "masked MoE E=16 max_m=256 N=7168 K=2048, UE8M0 scales",
}


def config(n: int) -> Workload:
    if n == 1:
        return dense(128, 256, 512, seed=1, outlier_frac=0.01, outlier_mult=50.0,
                     name="cfg1_dense_128x256x512")
    if n == 2:
        return dense(4096, 7168, 7168, seed=2, outlier_frac=0.001, outlier_mult=100.0,
                     name="cfg2_dense_4096x7168x7168")
    if n == 3:
        return dense(64, 24576, 1536, seed=3, w_std=0.02, name="cfg3_decode_64x24576x1536")
    if n == 4:
        return contiguous(8, 8192, 4096, 7168, seed=4, name="cfg4_contiguous_e8_t8192")
    if n == 5:
        return masked(16, 256, 7168, 2048, seed=5, ue8m0=True, name="cfg5_masked_e16_m256")
    raise ValueError(f"unknown configuration {n}")


def random_codes(rng: np.random.Generator, shape, allow_negative: bool = True) -> np.ndarray:
    """Uniformly random finite E4M3 bytes (the two NaN patterns excluded)."""
    c = rng.integers(0, 256, size=shape, dtype=np.uint8)
    nan = (c & 0x7F) == 0x7F
    c[nan] = 0x7E | (c[nan] & 0x80)
    if not allow_negative:
        c &= 0x7F
    return c


def random_pow2(rng: np.random.Generator, shape, lo: int = -12, hi: int = 4) -> np.ndarray:
    """Random powers of two 2^e, e uniform in [lo, hi], as float32."""
    e = rng.integers(lo, hi + 1, size=shape)
    return np.ldexp(np.ones(shape, np.float32), e).astype(np.float32)
