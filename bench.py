#!/usr/bin/env python3
"""Benchmark of the fine-grained block-scaled E4M3 GEMM hot path on one GPU.

    python bench.py [--steps K] [--warmup W] [--config 2|3|4|5] [--no-cpu-baseline] [--mx | --w4]

One step = one pass of the whole hot path over one batch of synthetic input:
1x128 activation quantization, 128x128 weight quantization and the
block-scaled GEMM (dense, contiguous-grouped or masked-grouped by workload).
Inputs are generated and moved to HBM before timing starts; outputs are
preallocated.  Prints ONE JSON line.

Default workload: dense prefill GEMM M=4096, N=7168, K=7168 (N(0,1) inputs,
0.1% of entries x100).  The other configurations are parity workloads that
can also be timed with --config.  --mx times the MXFP8 variant of a dense
workload instead: 1x32 E8M0 quantization of X and of W and the MXFP8 GEMM;
--w4 the MXFP4-weight variant: MXFP8 X, E2M1 W (1x32 E8M0 scales), their GEMM.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_FP8_TFLOPS = 5000.0      # MI355X dense FP8 MFMA
PEAK_HBM_GBS = 8000.0         # MI355X HBM3E
METRIC = "TFLOPS (and GB/s) of block-scaled FP8 GEMM; % of MI355X FP8 MFMA/HBM peak"


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the HIP sources, comments and blank space left out (they do not
    change the compiled kernels): counters taken for other sources are stale."""
    import re
    csrc = os.path.join(ROOT, "fine_grained_block_e4m3_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                src = f.read()
            src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
            src = re.sub(r"//[^\n]*", " ", src)
            src = " ".join(src.split())
            h.update(name.encode() + b"\0" + src.encode())
    return h.hexdigest()[:16]


def algorithmic_counts(wl):
    """Valid FLOPs and algorithmic bytes (A + sA + B + sB + Y, valid rows only,
    every weight byte once) of one GEMM launch."""
    import numpy as np
    K, N = wl.K, wl.N
    KB = K // 128
    if wl.kind == "dense":
        rows = wl.M
        w_rows = N
        n_sb = ((N + 127) // 128) * KB
    elif wl.kind == "contiguous":
        counts = np.bincount(wl.m_indices[wl.m_indices >= 0], minlength=wl.E)
        rows = int(counts.sum())
        used = int((counts > 0).sum())
        w_rows = used * N
        n_sb = used * (N // 128) * KB
    else:
        valid = np.clip(wl.masked_m, 0, wl.max_m)
        rows = int(valid.sum())
        used = int((valid > 0).sum())
        w_rows = used * N
        n_sb = used * (N // 128) * KB
    flops = 2.0 * rows * N * K
    nbytes = rows * K + 4 * rows * KB + w_rows * K + 4 * n_sb + 2 * rows * N
    return flops, float(nbytes), rows


def algorithmic_counts_mx(wl, w4: bool = False):
    """FLOPs and algorithmic bytes of one dense MXFP8 (or MXFP4-weight) GEMM
    launch: A + the 1x32 scale bytes of A + B (half a byte per element with
    E2M1 weights) + those of B + Y."""
    M, N, K = wl.M, wl.N, wl.K
    nbytes = M * K + M * (K // 32) + (N * K // 2 if w4 else N * K) + N * (K // 32) + 2 * M * N
    return 2.0 * M * N * K, float(nbytes), M


def load_traffic(key: str, sha: str):
    """HBM bytes per GEMM launch from committed rocprofv3 PMC counters, or None
    when they were taken for other kernel sources."""
    path = os.path.join(ROOT, "profiles", "counters.json")
    try:
        with open(path) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(key)
    if not e or e.get("source_sha") != sha:
        return None
    return float(e["hbm_bytes_per_dispatch"])


def cpu_baseline(wl, target_s: float, mx: bool = False, w4: bool = False):
    """Time the CPU oracle on a bounded sample of the same workload: the first
    Ms rows of X and first Ns rows of W, quantized and multiplied."""
    import numpy as np
    import oracle
    K = wl.K
    flags = oracle.FLAG_UE8M0 if wl.ue8m0 else 0

    def run(ms, ns):
        x = np.ascontiguousarray(wl.x[:ms])
        w = np.ascontiguousarray(wl.w[:ns])
        t0 = time.perf_counter()
        if w4:
            xq, ea = oracle.quant_mx(x)
            wq, eb = oracle.quant_mxfp4(w)
            oracle.gemm_mx_w4(xq, ea, wq, eb)
        elif mx:
            xq, ea = oracle.quant_mx(x)
            wq, eb = oracle.quant_mx(w)
            oracle.gemm_mx(xq, ea, wq, eb)
        else:
            xq, sa = oracle.quant_1x128(x, flags)
            wq, sb = oracle.quant_128x128(w, flags)
            oracle.gemm_nt(xq, sa, wq, sb, flags)
        return time.perf_counter() - t0

    # Grow the sample (rows of X first, then whole 128-row blocks of W) until
    # one run takes an eighth of the target, then size the timed sample from
    # that run's rate.
    M_cap, N_cap = min(wl.M, 4096), wl.w.shape[0]
    ms, ns = min(16, M_cap), min(128, N_cap)
    t = run(ms, ns)
    while t < target_s / 8 and (ms < M_cap or ns < N_cap):
        if ms < M_cap:
            ms = min(M_cap, 2 * ms)
        else:
            ns = min(N_cap, 2 * ns)
        t = run(ms, ns)
    scale = target_s / max(t, 1e-6)
    ms2 = int(min(M_cap, max(ms, ms * scale)))
    ns2 = int(min(N_cap, max(ns, (ns * scale * ms / ms2 + 64) // 128 * 128)))
    log(f"cpu baseline: {ms}x{ns} took {t:.2f}s; timing {ms2}x{ns2}x{K}")
    t2 = run(ms2, ns2)
    flops = 2.0 * ms2 * ns2 * K
    return {
        "value": flops / t2 / 1e12,
        "unit": "TFLOPS",
        "cores": oracle.num_threads(),
        "kind": "oracle",
        "sample": f"{wl.name}: X rows [0,{ms2}) and W rows [0,{ns2}), K={K}: oracle "
                  + ("quant_mx(X) + quant_mxfp4(W) + gemm_mx_w4" if w4 else
                     "quant_mx(X) + quant_mx(W) + gemm_mx" if mx else
                     "quant_1x128 + quant_128x128 + gemm_nt")
                  + f" ({flops:.3g} FLOP) in {t2:.2f} s",
        "seconds": t2,
        "cpu_model": _cpu_model(),
    }


def _cpu_model() -> str:
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor()


def copy_calibration(n_bytes: int = 1 << 30, reps: int = 3):
    """Plain device-to-device copies of a known size: the FETCH_SIZE /
    WRITE_SIZE counters of these dispatches give the scale from counter KiB to
    HBM bytes."""
    import torch
    src = torch.ones(n_bytes // 4, dtype=torch.float32, device="cuda")
    dst = torch.empty_like(src)
    for _ in range(reps):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes_read": n_bytes, "copy_bytes_written": n_bytes, "reps": reps}),
          flush=True)


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--shape", type=str, default=None,
                    help="M,N,K: a dense workload of that shape instead of --config, drawn like "
                         "configuration 3 (X ~ N(0,1), W ~ N(0, 0.02^2)); for decode-sized M")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-seconds", type=float, default=15.0)
    ap.add_argument("--mx", action="store_true",
                    help="the MXFP8 variant (1x32 E8M0 scales on both operands) of a dense workload")
    ap.add_argument("--w4", action="store_true",
                    help="MXFP8 activations with MXFP4 (E2M1) weights on a dense workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device copies (scale for HBM byte counters)")
    args = ap.parse_args()
    if args.copy_calibration:
        copy_calibration()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the multi-GPU path is not built", flush=True)
        sys.exit(2)

    import numpy as np
    import torch

    import fine_grained_block_e4m3_amd as fp8
    import workloads

    if not torch.cuda.is_available():
        print("bench.py needs a GPU", file=sys.stderr)
        sys.exit(1)
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    fp8.load_library()

    if args.shape:
        try:
            sM, sN, sK = (int(v) for v in args.shape.split(","))
        except ValueError:
            print("--shape takes M,N,K", file=sys.stderr)
            sys.exit(2)
        if min(sM, sN, sK) < 1 or sK % 128:
            print("--shape: M, N, K >= 1 and K a multiple of 128", file=sys.stderr)
            sys.exit(2)
        log(f"generating dense workload {sM}x{sN}x{sK}")
        wl = workloads.dense(sM, sN, sK, seed=3, w_std=0.02, name=f"dense_{sM}x{sN}x{sK}")
        traffic_key = f"shape_{sM}x{sN}x{sK}"
    else:
        log(f"generating workload {args.config}: {workloads.CONFIG_NAMES[args.config]}")
        wl = workloads.config(args.config)
        traffic_key = f"cfg{args.config}"
    ue8m0 = wl.ue8m0
    if (args.mx or args.w4) and wl.kind != "dense":
        print("--mx / --w4: dense workloads only (configs 1-3)", file=sys.stderr)
        sys.exit(2)
    mx = args.mx or args.w4
    x = torch.from_numpy(wl.x).to(dev)
    w = torch.from_numpy(wl.w).to(dev)
    M, K = wl.x.shape
    NW = wl.w.shape[0]
    xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
    sa = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
    wq = torch.empty((NW, K), dtype=torch.uint8, device=dev)
    sb = torch.empty(((NW + 127) // 128, K // 128), dtype=torch.float32, device=dev)
    if args.w4:
        ea = torch.empty((K // 128, M), dtype=torch.int32, device=dev)
        eb = torch.empty((K // 128, NW), dtype=torch.int32, device=dev)
        wq = torch.empty((NW, K // 2), dtype=torch.uint8, device=dev)
        y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)

        def gemm():
            fp8.gemm_nt_mx_w4(xq, ea, wq, eb, out=y)
    elif args.mx:
        ea = torch.empty((K // 128, M), dtype=torch.int32, device=dev)
        eb = torch.empty((K // 128, NW), dtype=torch.int32, device=dev)
        y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)

        def gemm():
            fp8.gemm_nt_mx(xq, ea, wq, eb, out=y)
    elif wl.kind == "dense":
        y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)

        def gemm():
            fp8.gemm_nt(xq, sa, wq, sb, ue8m0=ue8m0, out=y)
    elif wl.kind == "contiguous":
        y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)
        idx = torch.from_numpy(wl.m_indices).to(dev)
        wq3 = wq.view(wl.E, wl.N, K)
        sb3 = sb.view(wl.E, wl.N // 128, K // 128)

        def gemm():
            fp8.grouped_gemm_contiguous(xq, sa, wq3, sb3, idx, ue8m0=ue8m0, out=y)
    else:
        y = torch.empty((wl.E, wl.max_m, wl.N), dtype=torch.bfloat16, device=dev)
        mm = torch.from_numpy(wl.masked_m).to(dev)
        xq3 = xq.view(wl.E, wl.max_m, K)
        wq3 = wq.view(wl.E, wl.N, K)
        sb3 = sb.view(wl.E, wl.N // 128, K // 128)

        def gemm():
            fp8.grouped_gemm_masked(xq3, sa, wq3, sb3, mm, ue8m0=ue8m0, out=y)

    if mx:
        names = ("quant_mx_x", "quant_mxfp4_w" if args.w4 else "quant_mx_w", "gemm")

        def quant_x():
            fp8.quant_mx(x, out=(xq, ea))

        def quant_w():
            if args.w4:
                fp8.quant_mxfp4(w, out=(wq, eb))
            else:
                fp8.quant_mx(w, out=(wq, eb))
    else:
        names = ("quant_1x128", "quant_128x128", "gemm")

        def quant_x():
            fp8.quant_1x128(x, ue8m0=ue8m0, out=(xq, sa))

        def quant_w():
            fp8.quant_128x128(w, ue8m0=ue8m0, out=(wq, sb))
    stream = torch.cuda.current_stream(dev)

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        quant_x()
        if ev is not None:
            ev[1].record(stream)
        quant_w()
        if ev is not None:
            ev[2].record(stream)
        gemm()
        if ev is not None:
            ev[3].record(stream)

    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_kernel_ms = {n: float(np.mean([events[i][k].elapsed_time(events[i][k + 1])
                                       for i in range(args.steps)]))
                     for k, n in enumerate(names)}

    # The GEMM again on cold caches: before each launch a 1 GiB buffer (more
    # than the 256 MB MALL plus the L2s) is read, so that no operand comes
    # from a cache that the step's quantizers warmed.  A read leaves clean
    # lines, so no write-back of the flush is charged to the GEMM.  Reported
    # beside the in-pipeline figure that the roofline uses.
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    cold_ev = []
    for _ in range(min(args.steps, 20)):
        flush_buf.sum()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        gemm()
        b.record(stream)
        cold_ev.append((a, b))
    torch.cuda.synchronize()
    cold_ms = float(np.mean([a.elapsed_time(b) for a, b in cold_ev]))
    del flush_buf

    flops, nbytes, rows = algorithmic_counts_mx(wl, args.w4) if mx else algorithmic_counts(wl)
    gemm_s = per_kernel_ms["gemm"] / 1e3
    # ridge point of the roofline: peak FLOP/s over peak HBM bytes/s (625 FLOP/B)
    ridge = PEAK_FP8_TFLOPS * 1e12 / (PEAK_HBM_GBS * 1e9)
    compute_bound = wl.kind == "contiguous" or (wl.kind == "dense" and flops / nbytes > ridge)
    sha = kernel_source_sha()
    variant = "w4_" if args.w4 else ("mx_" if args.mx else "")
    traffic = load_traffic(f"gemm_{variant}{traffic_key}", sha)
    if compute_bound:
        achieved = flops / gemm_s / 1e12
        roof = {"bound": "mfma", "achieved": achieved, "peak": PEAK_FP8_TFLOPS,
                "unit": "TFLOP/s", "frac": achieved / PEAK_FP8_TFLOPS, "traffic": traffic}
    else:
        achieved = nbytes / gemm_s / 1e9
        roof = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS,
                "unit": "GB/s", "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    roof["kernel"] = "gemm"
    roof["avg_launch_us"] = per_kernel_ms["gemm"] * 1e3
    roof["algorithmic_flop"] = flops
    roof["algorithmic_bytes"] = nbytes

    if mx:
        qx_bytes = 4.0 * M * K + M * K + M * (K // 32)
        qw_bytes = 4.0 * NW * K + (NW * K // 2 if args.w4 else NW * K) + NW * (K // 32)
    else:
        qx_bytes = 4.0 * M * K + M * K + 4.0 * M * (K // 128)
        qw_bytes = 4.0 * NW * K + NW * K + 4.0 * sb.numel()
    kernels = {
        names[0]: {"avg_us": per_kernel_ms[names[0]] * 1e3,
                   "GB/s": qx_bytes / (per_kernel_ms[names[0]] / 1e3) / 1e9},
        names[1]: {"avg_us": per_kernel_ms[names[1]] * 1e3,
                   "GB/s": qw_bytes / (per_kernel_ms[names[1]] / 1e3) / 1e9},
        "gemm": {"avg_us": per_kernel_ms["gemm"] * 1e3, "TFLOPS": flops / gemm_s / 1e12,
                 "GB/s": nbytes / gemm_s / 1e9,
                 "frac_mfma": flops / gemm_s / 1e12 / PEAK_FP8_TFLOPS,
                 "frac_hbm": nbytes / gemm_s / 1e9 / PEAK_HBM_GBS},
    }

    kernels["gemm_cold_cache"] = {
        "avg_us": cold_ms * 1e3, "TFLOPS": flops / (cold_ms / 1e3) / 1e12,
        "GB/s": nbytes / (cold_ms / 1e3) / 1e9,
        "frac_mfma": flops / (cold_ms / 1e3) / 1e12 / PEAK_FP8_TFLOPS,
        "frac_hbm": nbytes / (cold_ms / 1e3) / 1e9 / PEAK_HBM_GBS,
        "flush": "a 1 GiB buffer read before each launch"}

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(wl, args.cpu_seconds, mx=args.mx, w4=args.w4)

    value = flops / (ms_per_step / 1e3) / 1e12
    cfg = {"workload": variant + wl.name, "kind": wl.kind, "M": int(M),
           "N": int(wl.N), "K": int(K), "valid_rows": rows,
           "scales": "mx_e8m0_1x32" if mx else ("ue8m0" if ue8m0 else "fp32"),
           "step": ("quant_mx(X) + quant_mxfp4(W) + MXFP8 x MXFP4 GEMM" if args.w4 else
                    "quant_mx(X) + quant_mx(W) + MXFP8 GEMM" if args.mx else
                    "quant_1x128(X) + quant_128x128(W) + block-scaled GEMM")}
    if wl.kind != "dense":
        cfg["experts"] = int(wl.E)
    out = {
        "metric": METRIC,
        "value": value,
        "unit": "TFLOPS",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": ms_per_step,
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8_e4m3 x fp4_e2m1" if args.w4 else "fp8_e4m3",
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "cpu_baseline": cpu,
        "kernels": kernels,
        "gpu": torch.cuda.get_device_name(dev),
        "kernel_source_sha": sha,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
