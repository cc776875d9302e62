#!/usr/bin/env python3
"""Benchmark of the fine-grained block-scaled E4M3 GEMM hot path on one GPU.

    python bench.py [--steps K] [--warmup W] [--config 2|3|4|5 | --shape M,N,K]
                    [--path exact|fast] [--mx | --w4] [--no-configs] [--no-cpu-baseline]

One step = one pass of the whole hot path over one batch of synthetic input:
1x128 activation quantization, 128x128 weight quantization and the
block-scaled GEMM (dense, contiguous-grouped or masked-grouped by workload).
Inputs are generated and moved to HBM before timing starts; outputs and
workspaces are preallocated.  Prints ONE JSON line.

Headline: the dense prefill GEMM M=4096, N=7168, K=7168 (N(0,1) inputs, 0.1%
of entries x100) on the default path -- exact E4M3 products (converted to
FP16 and multiplied by the FP16 matrix instruction, which keeps the full
product and sums it in FP32), promoted with sA*sB every 128-K block.  The
step is timed warm (K steps back to back) and, as a second figure, with
caches flushed before every step.  Besides the headline the line carries:
  - opt_in_fast_accum: the same GEMM with FP8_FLAG_FAST_ACCUM (block partials
    from the FP8 matrix instruction; documented error bound, not the default);
  - configs: GEMM-only records of the decode, contiguous-MoE and masked-MoE
    workloads (and the prefill one) on both paths, with bound, roofline
    fraction and, where rocprofv3 counters for these kernel sources are
    committed, the HBM-traffic ratio;
  - clock: the GPU clock sampled while the GEMM runs back to back;
  - cpu_baseline: the CPU oracle on a bounded sample, quantization and GEMM
    seconds apart, at the default thread count and on one thread.
--mx times the MXFP8 variant of a dense workload instead (1x32 E8M0
quantization of X and W, MXFP8 GEMM); --w4 MXFP8 activations with MXFP4
(E2M1) weights.  --gpus above 1 exits: this benchmark runs on one GPU.
"""
from __future__ import annotations

import argparse
import hashlib
import json
import os
import platform
import sys
import threading
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)

PEAK_TFLOPS = {"f16": 2500.0, "fp8": 5000.0}   # MI355X dense MFMA peaks
PEAK_HBM_GBS = 8000.0                            # MI355X HBM3E
METRIC = "TFLOPS (and GB/s) of block-scaled FP8 GEMM; % of MI355X FP8 MFMA/HBM peak"
FLAG_FAST_ACCUM = 2


def log(*a):
    print(*a, file=sys.stderr, flush=True)


def kernel_source_sha() -> str:
    """Hash of the HIP sources, comments and blank space left out (they do not
    change the compiled kernels): counters taken for other sources are stale."""
    import re
    csrc = os.path.join(ROOT, "fine_grained_block_e4m3_amd", "csrc")
    h = hashlib.sha256()
    for name in sorted(os.listdir(csrc)):
        if name.endswith((".h", ".hip", ".inc")):
            with open(os.path.join(csrc, name), encoding="utf-8") as f:
                src = f.read()
            src = re.sub(r"/\*.*?\*/", " ", src, flags=re.S)
            src = re.sub(r"//[^\n]*", " ", src)
            src = " ".join(src.split())
            h.update(name.encode() + b"\0" + src.encode())
    return h.hexdigest()[:16]


def stats(xs):
    import numpy as np
    a = np.asarray(xs, dtype=np.float64)
    return {"mean": float(a.mean()), "median": float(np.median(a)), "min": float(a.min()), "n": int(a.size)}


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


def load_counters(key: str, sha: str):
    """The committed rocprofv3 PMC record of one GEMM kernel, or None when it
    was taken for other kernel sources."""
    try:
        with open(os.path.join(ROOT, "profiles", "counters.json")) as f:
            data = json.load(f)
    except (OSError, ValueError):
        return None
    e = data.get(key)
    if not e or e.get("source_sha") != sha:
        return None
    return e


def roofline(flops, nbytes, seconds, peak_key, compute_bound, counters):
    traffic = float(counters["hbm_bytes_per_dispatch"]) if counters else None
    if compute_bound:
        achieved = flops / seconds / 1e12
        peak = PEAK_TFLOPS[peak_key]
        r = {"bound": "mfma", "achieved": achieved, "peak": peak, "unit": "TFLOP/s",
             "frac": achieved / peak, "traffic": traffic, "mfma_dtype": peak_key}
        if peak_key != "fp8":
            r["frac_of_fp8_peak"] = achieved / PEAK_TFLOPS["fp8"]
    else:
        achieved = nbytes / seconds / 1e9
        r = {"bound": "hbm", "achieved": achieved, "peak": PEAK_HBM_GBS, "unit": "GB/s",
             "frac": achieved / PEAK_HBM_GBS, "traffic": traffic}
    r["traffic_ratio"] = traffic / nbytes if traffic else None
    if counters and counters.get("clock_mhz_grbm"):
        r["clock_mhz_counters"] = counters["clock_mhz_grbm"]
    if counters and counters.get("mfma_busy_frac") is not None:
        r["mfma_busy_frac_counters"] = counters["mfma_busy_frac"]
    return r


def _cpu_model() -> dict:
    info = {}
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                k, _, v = line.partition(":")
                k = k.strip()
                if k in ("model name", "vendor_id", "cpu family", "model", "stepping", "cpu MHz") \
                        and k not in info:
                    info[k] = v.strip()
                if len(info) == 6:
                    break
    except OSError:
        pass
    info.setdefault("model name", platform.processor())
    return info


def cpu_baseline(wl, target_s: float, mx: bool = False, w4: bool = False):
    """Time the CPU oracle on a bounded sample of the same workload: the first
    ms rows of X and the first ns rows of W, quantized and multiplied, the
    quantization and the GEMM timed apart; then the same at one thread on a
    sample a quarter of the size (the per-core figure)."""
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
        elif mx:
            xq, ea = oracle.quant_mx(x)
            wq, eb = oracle.quant_mx(w)
        else:
            xq, sa = oracle.quant_1x128(x, flags)
            wq, sb = oracle.quant_128x128(w, flags)
        t1 = time.perf_counter()
        if w4:
            oracle.gemm_mx_w4(xq, ea, wq, eb)
        elif mx:
            oracle.gemm_mx(xq, ea, wq, eb)
        else:
            oracle.gemm_nt(xq, sa, wq, sb, flags)
        t2 = time.perf_counter()
        return t1 - t0, t2 - t1

    def sized(target):
        # Grow the sample (rows of X first, then whole 128-row blocks of W)
        # until one run takes an eighth of the target, then size the timed
        # sample from that run's rate.
        M_cap, N_cap = min(wl.M, 4096), wl.w.shape[0]
        ms, ns = min(16, M_cap), min(128, N_cap)
        t = sum(run(ms, ns))
        while t < target / 8 and (ms < M_cap or ns < N_cap):
            if ms < M_cap:
                ms = min(M_cap, 2 * ms)
            else:
                ns = min(N_cap, 2 * ns)
            t = sum(run(ms, ns))
        scale = target / max(t, 1e-6)
        ms2 = int(min(M_cap, max(ms, ms * scale)))
        ns2 = int(min(N_cap, max(ns, (ns * scale * ms / ms2 + 64) // 128 * 128)))
        tq, tg = run(ms2, ns2)
        if tq + tg < target / 2 and (ms2 < M_cap or ns2 < N_cap):
            scale = target / (tq + tg)
            ms3 = int(min(M_cap, ms2 * scale))
            ns3 = int(min(N_cap, max(ns2, (ns2 * scale * ms2 / max(ms3, 1) + 64) // 128 * 128)))
            ms2, ns2 = max(ms2, ms3), ns3
            tq, tg = run(ms2, ns2)
        return ms2, ns2, tq, tg

    what = ("quant_mx(X) + quant_mxfp4(W) + gemm_mx_w4" if w4 else
            "quant_mx(X) + quant_mx(W) + gemm_mx" if mx else
            "quant_1x128(X) + quant_128x128(W) + gemm_nt")
    threads = oracle.num_threads()
    ms, ns, tq, tg = sized(target_s)
    flops = 2.0 * ms * ns * K
    log(f"cpu baseline ({threads} threads): {ms}x{ns}x{K} quant {tq:.2f}s gemm {tg:.2f}s")
    oracle.set_num_threads(1)
    try:
        ms1, ns1, tq1, tg1 = sized(max(target_s / 4, 1.0))
    finally:
        oracle.set_num_threads(threads)
    flops1 = 2.0 * ms1 * ns1 * K
    log(f"cpu baseline (1 thread): {ms1}x{ns1}x{K} quant {tq1:.2f}s gemm {tg1:.2f}s")
    try:
        affinity = len(os.sched_getaffinity(0))
    except (AttributeError, OSError):
        affinity = None
    return {
        "value": flops / (tq + tg) / 1e12,
        "unit": "TFLOPS",
        "cores": threads,
        "kind": "oracle",
        "sample": f"{wl.name}: X rows [0,{ms}) and W rows [0,{ns}), K={K}: oracle {what} "
                  f"({flops:.3g} FLOP) in {tq + tg:.2f} s on {threads} threads",
        "quant_seconds": tq,
        "gemm_seconds": tg,
        "gemm_tflops": flops / tg / 1e12,
        "one_thread": {"value": flops1 / (tq1 + tg1) / 1e12, "unit": "TFLOPS",
                       "quant_seconds": tq1, "gemm_seconds": tg1,
                       "gemm_tflops": flops1 / tg1 / 1e12,
                       "sample": f"X rows [0,{ms1}) and W rows [0,{ns1}), K={K}, 1 thread"},
        "nproc": os.cpu_count(),
        "affinity_cpus": affinity,
        "omp_num_threads_env": os.environ.get("OMP_NUM_THREADS"),
        "cpu": _cpu_model(),
    }


def _num(v):
    if isinstance(v, (list, tuple)):
        vals = [float(x) for x in v if isinstance(x, (int, float)) and 0 < x < 10000]
        return sum(vals) / len(vals) if vals else None
    return float(v) if isinstance(v, (int, float)) and 0 <= v < 10000 else None


def clock_sampler_main():
    """`bench.py --clock-sampler`: a child process that reads the GPU's
    graphics clock through amd-smi (it never opens the GPU for compute).
    Waits for "start <PCI address>" on stdin, picks the amd-smi device with
    that address (the host may show amd-smi more GPUs than the one this
    benchmark runs on), samples every 2 ms until "stop", then prints one JSON
    object of samples."""
    import select
    out = {"samples": [], "error": None, "bdf": None, "devices": 0}
    try:
        import amdsmi
        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        out["devices"] = len(handles)
    except Exception as e:                      # monitoring is optional: report why it is missing
        handles, out["error"] = [], f"{type(e).__name__}: {e}"[:200]
    sys.stdout.write("ready\n")
    sys.stdout.flush()
    cmd = sys.stdin.readline().split()
    if not cmd or cmd[0] != "start":
        return
    want = cmd[1].lower() if len(cmd) > 1 else ""
    h = None
    try:
        for hh in handles:
            if want and amdsmi.amdsmi_get_gpu_device_bdf(hh).lower().startswith(want):
                h = hh
        if h is None and len(handles) == 1:
            h = handles[0]
        if h is not None:
            out["bdf"] = amdsmi.amdsmi_get_gpu_device_bdf(h)
        else:
            seen = [amdsmi.amdsmi_get_gpu_device_bdf(hh) for hh in handles[:16]]
            out["error"] = f"no amd-smi device at {want or '?'} among {seen}"[:200]
    except Exception as e:
        out["error"] = f"{type(e).__name__}: {e}"[:200]
    while True:
        if select.select([sys.stdin], [], [], 0.002)[0]:
            break
        if h is None:
            continue
        smp = {"t": time.perf_counter()}
        try:
            info = amdsmi.amdsmi_get_clock_info(h, amdsmi.AmdSmiClkType.SYS)
            smp["clk_info_mhz"] = _num(info.get("clk"))
            smp["max_mhz"] = _num(info.get("max_clk"))
        except Exception as e:
            out["error"] = f"clock_info: {type(e).__name__}: {e}"[:200]
        try:
            m = amdsmi.amdsmi_get_gpu_metrics_info(h)
            smp["current_gfxclks_mhz"] = _num(m.get("current_gfxclks"))
            smp["current_gfxclk_mhz"] = _num(m.get("current_gfxclk"))
            smp["average_gfxclk_mhz"] = _num(m.get("average_gfxclk_frequency"))
            smp["gfx_activity_pct"] = _num(m.get("average_gfx_activity"))
        except Exception as e:
            out["error"] = f"gpu_metrics: {type(e).__name__}: {e}"[:200]
        out["samples"].append(smp)
    sys.stdout.write(json.dumps(out) + "\n")
    sys.stdout.flush()


class ClockSampler:
    """The graphics clock read through amd-smi while work runs, from a child
    process (`bench.py --clock-sampler`) started before this process touches
    the GPU, so that neither the interpreter lock nor a fork after GPU
    initialisation stands in the way."""

    def __init__(self):
        import subprocess
        self.err = None
        try:
            self.proc = subprocess.Popen([sys.executable, os.path.abspath(__file__), "--clock-sampler"],
                                         stdin=subprocess.PIPE, stdout=subprocess.PIPE, text=True)
            if self.proc.stdout.readline().strip() != "ready":
                raise RuntimeError("sampler did not start")
        except Exception as e:
            self.proc, self.err = None, f"{type(e).__name__}: {e}"[:200]

    def during(self, launch, n_launch, sync, bdf=""):
        """Sample while n_launch back-to-back launches run on the GPU at PCI
        address bdf; report the medians over the samples taken while the
        graphics activity read 50% or more (all samples past the first quarter
        if it is missing)."""
        if self.proc is None:
            return {"mhz": None, "error": self.err}
        try:
            self.proc.stdin.write(f"start {bdf}\n")
            self.proc.stdin.flush()
            for _ in range(n_launch):
                launch()
            sync()
            self.proc.stdin.write("stop\n")
            self.proc.stdin.flush()
            res = json.loads(self.proc.stdout.readline())
            self.proc.wait(timeout=10)
        except Exception as e:
            return {"mhz": None, "error": f"{type(e).__name__}: {e}"[:200]}
        samples = res["samples"]
        busy = [s for s in samples if (s.get("gfx_activity_pct") or 0) >= 50]
        use = busy or samples[len(samples) // 4:] or samples
        out = {"samples": len(samples), "busy_samples": len(busy), "bdf": res.get("bdf"),
               "amd_smi_devices": res.get("devices"),
               "source": "amd-smi in a child process, sampled every 2 ms", "error": res.get("error")}
        for key in ("current_gfxclks_mhz", "current_gfxclk_mhz", "average_gfxclk_mhz", "clk_info_mhz",
                    "gfx_activity_pct", "max_mhz"):
            vals = [s[key] for s in use if s.get(key) is not None]
            out[key] = stats(vals)["median"] if vals else None
        out["mhz"] = next((out[k] for k in ("current_gfxclks_mhz", "current_gfxclk_mhz",
                                             "average_gfxclk_mhz", "clk_info_mhz") if out[k]), None)
        return out

    def close(self):
        if self.proc is not None and self.proc.poll() is None:
            try:
                self.proc.stdin.close()
                self.proc.wait(timeout=10)
            except Exception:
                self.proc.kill()


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


class Problem:
    """Device buffers of one workload and closures that launch its kernels."""

    def __init__(self, wl, dev, mx=False, w4=False):
        import torch
        import fine_grained_block_e4m3_amd as fp8
        self.wl, self.mx, self.w4 = wl, mx or w4, w4
        self.fp8 = fp8
        x = torch.from_numpy(wl.x).to(dev)
        w = torch.from_numpy(wl.w).to(dev)
        self.x, self.w = x, w
        M, K = wl.x.shape
        NW = wl.w.shape[0]
        self.M, self.K, self.NW = M, K, NW
        ue8m0 = wl.ue8m0
        self.xq = torch.empty((M, K), dtype=torch.uint8, device=dev)
        if self.mx:
            self.ea = torch.empty((K // 128, M), dtype=torch.int32, device=dev)
            self.eb = torch.empty((K // 128, NW), dtype=torch.int32, device=dev)
            self.wq = torch.empty((NW, K // 2 if w4 else K), dtype=torch.uint8, device=dev)
            self.quant_x = lambda: fp8.quant_mx(x, out=(self.xq, self.ea))
            if w4:
                self.quant_w = lambda: fp8.quant_mxfp4(w, out=(self.wq, self.eb))
                self.names = ("quant_mx_x", "quant_mxfp4_w", "gemm")
            else:
                self.quant_w = lambda: fp8.quant_mx(w, out=(self.wq, self.eb))
                self.names = ("quant_mx_x", "quant_mx_w", "gemm")
        else:
            self.sa = torch.empty((K // 128, M), dtype=torch.float32, device=dev)
            self.wq = torch.empty((NW, K), dtype=torch.uint8, device=dev)
            self.sb = torch.empty(((NW + 127) // 128, K // 128), dtype=torch.float32, device=dev)
            self.quant_x = lambda: fp8.quant_1x128(x, ue8m0=ue8m0, out=(self.xq, self.sa))
            self.quant_w = lambda: fp8.quant_128x128(w, ue8m0=ue8m0, out=(self.wq, self.sb))
            self.names = ("quant_1x128", "quant_128x128", "gemm")
        if wl.kind == "masked":
            self.y = torch.empty((wl.E, wl.max_m, wl.N), dtype=torch.bfloat16, device=dev)
            self.mm = torch.from_numpy(wl.masked_m).to(dev)
        else:
            self.y = torch.empty((M, wl.N), dtype=torch.bfloat16, device=dev)
        if wl.kind == "contiguous":
            self.idx = torch.from_numpy(wl.m_indices).to(dev)
        self.ws = {}
        if wl.kind == "dense" and not self.mx:
            L = fp8.load_library()
            for fast in (False, True):
                nb = int(L.fp8_gemm_workspace_size(M, wl.N, K, (1 if ue8m0 else 0) |
                                                   (FLAG_FAST_ACCUM if fast else 0)))
                self.ws[fast] = torch.empty(max(nb, 1), dtype=torch.uint8, device=dev) if nb else None

    def gemm_fn(self, fast: bool):
        fp8, wl, K = self.fp8, self.wl, self.K
        ue8m0 = wl.ue8m0
        if self.w4:
            return lambda: fp8.gemm_nt_mx_w4(self.xq, self.ea, self.wq, self.eb, out=self.y)
        if self.mx:
            return lambda: fp8.gemm_nt_mx(self.xq, self.ea, self.wq, self.eb, out=self.y)
        if wl.kind == "dense":
            ws = self.ws.get(fast)
            return lambda: fp8.gemm_nt(self.xq, self.sa, self.wq, self.sb, ue8m0=ue8m0,
                                       fast_accum=fast, out=self.y, workspace=ws)
        if wl.kind == "contiguous":
            wq3 = self.wq.view(wl.E, wl.N, K)
            sb3 = self.sb.view(wl.E, wl.N // 128, K // 128)
            return lambda: fp8.grouped_gemm_contiguous(self.xq, self.sa, wq3, sb3, self.idx,
                                                       ue8m0=ue8m0, fast_accum=fast, out=self.y)
        xq3 = self.xq.view(wl.E, wl.max_m, K)
        wq3 = self.wq.view(wl.E, wl.N, K)
        sb3 = self.sb.view(wl.E, wl.N // 128, K // 128)
        return lambda: fp8.grouped_gemm_masked(xq3, self.sa, wq3, sb3, self.mm, ue8m0=ue8m0,
                                               fast_accum=fast, out=self.y)

    def counts(self):
        return algorithmic_counts_mx(self.wl, self.w4) if self.mx else algorithmic_counts(self.wl)


def time_each(fn, reps, stream, flush=None):
    """Per-launch durations (ms) from HIP events recorded on the launch stream
    right before and after each launch; with `flush`, it runs (untimed)
    before each launch."""
    import torch
    ev = []
    for _ in range(reps):
        if flush is not None:
            flush()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(stream)
        fn()
        b.record(stream)
        ev.append((a, b))
    torch.cuda.synchronize()
    return [a.elapsed_time(b) for a, b in ev]


def time_batched(fn, reps, stream):
    """Average duration (ms) of `reps` launches queued back to back between two
    events: no host gap between launches."""
    import torch
    a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    a.record(stream)
    for _ in range(reps):
        fn()
    b.record(stream)
    torch.cuda.synchronize()
    return a.elapsed_time(b) / reps


def launch_plan(prob, fast):
    """The kernel launches one GEMM call of the workload makes (the library's
    host-side plan): the timed figures cover all of them."""
    import torch
    wl = prob.wl
    cus = torch.cuda.get_device_properties(torch.cuda.current_device()).multi_processor_count
    M = wl.max_m if wl.kind == "masked" else prob.M
    pl = prob.fp8.gemm_plan(wl.kind, M, wl.N, prob.K, ue8m0=wl.ue8m0, fast_accum=fast,
                            mx=prob.mx, compute_units=cus)
    kind = {0: "tile", 1: "decode", 2: "decode_x", 3: "exact_decode", 4: "exact_decode_x"}[pl["kernel"]]
    out = {"launches": 1, "main": f"{kind} {pl['tile_m']}x{pl['tile_n']}, {pl['tiles']} tiles, grid {pl['grid']}"
                                   + (" per expert" if wl.kind == "masked" else "")}
    if pl["paired"]:
        # contiguous pair schedule: the launches split the blocks on the device
        out["launches"] = 3
        out["main"] = (f"tile {pl['tile_m']}x{pl['tile_n']} over pairs of one expert's 128-row blocks, "
                       f"at most {pl['tiles']} tiles, grid {pl['grid']}")
        out["mid"] = f"tile {pl['mid_tile_m']}x{pl['mid_tile_n']} over the blocks left, at most {pl['mid_tiles']} tiles"
        out["tail"] = (f"tile {pl['tail_tile_m']}x{pl['tail_tile_n']} over the blocks the middle launch leaves, "
                       f"at most {pl['tail_tiles']} tiles")
    elif pl["tail_tiles"]:
        out["launches"] = 2
        where = (f"rows [{pl['main_rows']}, {prob.M})" if wl.kind == "contiguous"
                 else f"columns [{pl['main_cols']}, {wl.N})")
        out["tail"] = f"tile {pl['tail_tile_m']}x{pl['tail_tile_n']}, {pl['tail_tiles']} tiles, {where}"
    return out


def gemm_record(prob, fast, stream, sha, key, reps=20):
    """GEMM-only timing of one workload on one path, with its roofline."""
    import torch
    fn = prob.gemm_fn(fast)
    for _ in range(3):
        fn()
    torch.cuda.synchronize()
    each = stats([t * 1e3 for t in time_each(fn, reps, stream)])
    batched_us = time_batched(fn, reps, stream) * 1e3
    flops, nbytes, rows = prob.counts()
    wl = prob.wl
    peak_key = "fp8" if (fast or prob.mx) else "f16"
    ridge = PEAK_TFLOPS[peak_key] * 1e12 / (PEAK_HBM_GBS * 1e9)
    compute_bound = wl.kind == "contiguous" or (wl.kind == "dense" and flops / nbytes > ridge)
    counters = load_counters(key, sha)
    r = {"workload": wl.name, "path": "fast_accum" if fast else "default",
         "avg_us": each["mean"], "median_us": each["median"], "min_us": each["min"],
         "batched_avg_us": batched_us,
         "TFLOPS": flops / (each["mean"] / 1e6) / 1e12, "GB/s": nbytes / (each["mean"] / 1e6) / 1e9}
    r.update(roofline(flops, nbytes, each["mean"] / 1e6, peak_key, compute_bound, counters))
    r["algorithmic_flop"], r["algorithmic_bytes"] = flops, nbytes
    if not prob.mx:
        r["launch_plan"] = launch_plan(prob, fast)
    if counters:
        r["kernel_trace_avg_us"] = counters.get("avg_us_kernel_trace")
    return r


def main():
    ap = argparse.ArgumentParser(description=__doc__, formatter_class=argparse.RawTextHelpFormatter)
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", type=int, default=2, choices=[1, 2, 3, 4, 5])
    ap.add_argument("--shape", type=str, default=None,
                    help="M,N,K: a dense workload of that shape instead of --config, drawn like "
                         "configuration 3 (X ~ N(0,1), W ~ N(0, 0.02^2)); for decode-sized M")
    ap.add_argument("--path", choices=["exact", "fast"], default="exact",
                    help="GEMM path of the timed step: exact (default) or FP8_FLAG_FAST_ACCUM")
    ap.add_argument("--no-configs", action="store_true",
                    help="skip the GEMM-only records of the other workloads")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the clock sampling (half a second of back-to-back GEMM launches)")
    ap.add_argument("--cpu-seconds", type=float, default=12.0)
    ap.add_argument("--mx", action="store_true",
                    help="the MXFP8 variant (1x32 E8M0 scales on both operands) of a dense workload")
    ap.add_argument("--w4", action="store_true",
                    help="MXFP8 activations with MXFP4 (E2M1) weights on a dense workload")
    ap.add_argument("--copy-calibration", action="store_true",
                    help="only run plain 1 GiB device copies (scale for HBM byte counters)")
    ap.add_argument("--clock-sampler", action="store_true", help=argparse.SUPPRESS)
    args = ap.parse_args()
    if args.clock_sampler:
        clock_sampler_main()
        return
    if args.copy_calibration:
        copy_calibration()
        return

    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py runs on exactly one GPU (asked for --gpus {args.gpus}, "
              f"WORLD_SIZE={world}); the multi-GPU path is not built", flush=True)
        sys.exit(2)
    if args.steps < 1 or args.warmup < 0:
        print("--steps >= 1 and --warmup >= 0", file=sys.stderr)
        sys.exit(2)

    # the clock sampler starts before this process touches the GPU
    sampler = None if args.no_clock else ClockSampler()

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
        tkey = f"shape_{sM}x{sN}x{sK}"
    else:
        log(f"generating workload {args.config}: {workloads.CONFIG_NAMES[args.config]}")
        wl = workloads.config(args.config)
        tkey = f"cfg{args.config}"
    if (args.mx or args.w4) and wl.kind != "dense":
        print("--mx / --w4: dense workloads only (configs 1-3)", file=sys.stderr)
        sys.exit(2)
    mx = args.mx or args.w4
    fast = args.path == "fast"
    variant = "w4" if args.w4 else ("mx" if args.mx else ("fast" if fast else "exact"))
    prob = Problem(wl, dev, mx=args.mx, w4=args.w4)
    gemm = prob.gemm_fn(fast)
    names = prob.names
    stream = torch.cuda.current_stream(dev)
    sha = kernel_source_sha()

    def step(ev=None):
        if ev is not None:
            ev[0].record(stream)
        prob.quant_x()
        if ev is not None:
            ev[1].record(stream)
        prob.quant_w()
        if ev is not None:
            ev[2].record(stream)
        gemm()
        if ev is not None:
            ev[3].record(stream)

    # ---- timed region: K warm steps back to back ----------------------------
    log(f"warmup {args.warmup} steps")
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    events = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(args.steps)]
    log(f"timing {args.steps} steps ({variant} path)")
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for i in range(args.steps):
        step(events[i])
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    per_kernel = {n: stats([events[i][k].elapsed_time(events[i][k + 1]) * 1e3
                            for i in range(args.steps)])
                  for k, n in enumerate(names)}
    step_us = stats([events[i][0].elapsed_time(events[i][3]) * 1e3 for i in range(args.steps)])

    # ---- the same step with every cache flushed before it -------------------
    # A 1 GiB read (more than the 256 MB MALL and the L2s together) runs before
    # each step, outside its events: no operand or scale comes from a cache
    # warmed by the previous step.  A read leaves clean lines, so no
    # write-back of the flush is charged to the step.
    flush_buf = torch.ones(1 << 28, dtype=torch.float32, device=dev)
    n_flush = min(args.steps, 20)
    fev = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_flush)]
    for i in range(n_flush):
        flush_buf.sum()
        step(fev[i])
    torch.cuda.synchronize()
    flushed_step = stats([fev[i][0].elapsed_time(fev[i][3]) * 1e3 for i in range(n_flush)])
    flushed_gemm = stats([fev[i][2].elapsed_time(fev[i][3]) * 1e3 for i in range(n_flush)])
    del flush_buf

    # ---- GPU clock while the GEMM runs back to back (about half a second) ---
    clock = None
    if sampler is not None:
        n_clock = int(min(4000, max(50, 0.5e6 / max(per_kernel["gemm"]["mean"], 1.0))))
        props = torch.cuda.get_device_properties(dev)
        bdf = "{:04x}:{:02x}:{:02x}".format(getattr(props, "pci_domain_id", 0), getattr(props, "pci_bus_id", 0),
                                            getattr(props, "pci_device_id", 0))
        clock = sampler.during(gemm, n_clock, torch.cuda.synchronize, bdf)
        clock["while"] = f"{n_clock} back-to-back launches of the {variant} GEMM on {wl.name}"
        sampler.close()

    flops, nbytes, rows = prob.counts()
    gemm_s = per_kernel["gemm"]["mean"] / 1e6
    peak_key = "fp8" if (fast or mx) else "f16"
    ridge = PEAK_TFLOPS[peak_key] * 1e12 / (PEAK_HBM_GBS * 1e9)
    compute_bound = wl.kind == "contiguous" or (wl.kind == "dense" and flops / nbytes > ridge)
    roof = roofline(flops, nbytes, gemm_s, peak_key, compute_bound,
                    load_counters(f"gemm_{variant}_{tkey}", sha))
    roof["kernel"] = "gemm"
    roof["avg_launch_us"] = per_kernel["gemm"]["mean"]
    if not mx:
        # avg_launch_us spans the GEMM call: every launch of this plan
        roof["launch_plan"] = launch_plan(prob, fast)
    roof["algorithmic_flop"] = flops
    roof["algorithmic_bytes"] = nbytes
    roof["flushed_avg_launch_us"] = flushed_gemm["mean"]
    roof["flushed_frac"] = roof["frac"] * per_kernel["gemm"]["mean"] / flushed_gemm["mean"]

    if mx:
        qx_bytes = 4.0 * prob.M * prob.K + prob.M * prob.K + prob.M * (prob.K // 32)
        qw_bytes = 4.0 * prob.NW * prob.K + prob.wq.numel() + prob.NW * (prob.K // 32)
    else:
        qx_bytes = 4.0 * prob.M * prob.K + prob.M * prob.K + 4.0 * prob.sa.numel()
        qw_bytes = 4.0 * prob.NW * prob.K + prob.NW * prob.K + 4.0 * prob.sb.numel()
    kernels = {
        names[0]: {**{k + "_us": v for k, v in per_kernel[names[0]].items() if k != "n"},
                   "GB/s": qx_bytes / (per_kernel[names[0]]["mean"] / 1e6) / 1e9},
        names[1]: {**{k + "_us": v for k, v in per_kernel[names[1]].items() if k != "n"},
                   "GB/s": qw_bytes / (per_kernel[names[1]]["mean"] / 1e6) / 1e9},
        "gemm": {**{k + "_us": v for k, v in per_kernel["gemm"].items() if k != "n"},
                 "TFLOPS": flops / gemm_s / 1e12, "GB/s": nbytes / gemm_s / 1e9},
    }

    # ---- the opt-in FP8-instruction path on the same workload ----------------
    fast_rec = None
    if not mx and not fast:
        fast_rec = gemm_record(prob, True, stream, sha, f"gemm_fast_{tkey}")
        fast_rec["note"] = ("FP8_FLAG_FAST_ACCUM: block partials from the FP8 matrix instruction, "
                            "which truncates products inside 8-wide K groups; not the default path")

    # ---- GEMM-only records of the other workloads ----------------------------
    configs = {}
    if not args.no_configs and not args.shape and not mx and args.config == 2:
        configs["cfg2"] = {"default": gemm_record(prob, False, stream, sha, "gemm_exact_cfg2"),
                           "fast_accum": fast_rec}
    cpu_wl = wl
    del prob, gemm
    torch.cuda.empty_cache()
    if not args.no_configs and not args.shape and not mx and args.config == 2:
        for c in (3, 4, 5):
            log(f"generating workload {c}: {workloads.CONFIG_NAMES[c]}")
            wc = workloads.config(c)
            pc = Problem(wc, dev)
            pc.quant_x()
            pc.quant_w()
            torch.cuda.synchronize()
            configs[f"cfg{c}"] = {
                "default": gemm_record(pc, False, stream, sha, f"gemm_exact_cfg{c}"),
                "fast_accum": gemm_record(pc, True, stream, sha, f"gemm_fast_cfg{c}")}
            del pc, wc
            torch.cuda.empty_cache()

    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(cpu_wl, args.cpu_seconds, mx=args.mx, w4=args.w4)

    value = flops / (ms_per_step / 1e3) / 1e12
    cfg = {"workload": ("" if variant in ("exact", "fast") else variant + "_") + wl.name,
           "kind": wl.kind, "M": int(wl.x.shape[0]), "N": int(wl.N), "K": int(wl.K), "valid_rows": rows,
           "scales": "mx_e8m0_1x32" if mx else ("ue8m0" if wl.ue8m0 else "fp32"),
           "gemm_path": {"exact": "default (exact E4M3 products, FP32 block partials)",
                         "fast": "FP8_FLAG_FAST_ACCUM (FP8 matrix instruction partials)",
                         "mx": "MXFP8", "w4": "MXFP8 x MXFP4"}[variant],
           "step": ("quant_mx(X) + quant_mxfp4(W) + MXFP8 x MXFP4 GEMM" if args.w4 else
                    "quant_mx(X) + quant_mx(W) + MXFP8 GEMM" if args.mx else
                    "quant_1x128(X) + quant_128x128(W) + block-scaled GEMM")}
    if wl.kind != "dense":
        cfg["experts"] = int(wl.E)
    dtype = {"exact": "fp8_e4m3 operands; f16 MFMA products (exact), f32 accumulation",
             "fast": "fp8_e4m3 (fp8 MFMA), f32 accumulation",
             "mx": "fp8_e4m3 (scaled fp8 MFMA), f32 accumulation",
             "w4": "fp8_e4m3 x fp4_e2m1 (scaled MFMA), f32 accumulation"}[variant]
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
        "dtype": dtype,
        "data": "synthetic",
        "config": cfg,
        "roofline": roof,
        "cpu_baseline": cpu,
        "step_us": step_us,
        "flushed": {"step_us": flushed_step, "gemm_us": flushed_gemm,
                    "value": flops / (flushed_step["mean"] / 1e6) / 1e12,
                    "flush": "a 1 GiB device buffer read before each step, outside its events"},
        "kernels": kernels,
        "opt_in_fast_accum": fast_rec,
        "configs": configs,
        "clock": clock,
        "gpu": torch.cuda.get_device_name(dev),
        "kernel_source_sha": sha,
    }
    print(json.dumps(out), flush=True)


if __name__ == "__main__":
    main()
