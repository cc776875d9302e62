"""Build libfp8gemm.so (HIP, gfx950 only) in-tree.

    python -m fine_grained_block_e4m3_amd.build [--asm]

The library is compiled ahead of time with hipcc; there is no runtime JIT.
"""
from __future__ import annotations

import os
import subprocess
import sys

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
LIB = os.path.join(HERE, "libfp8gemm.so")
SOURCES = [os.path.join(CSRC, "fp8gemm_api.hip")]
ARCH = "gfx950"

HIPCC_FLAGS = [
    f"--offload-arch={ARCH}",
    "-O3",
    "-std=c++17",
    "-fPIC",
    "-shared",
    # packed FP32 VALU forms are kept out of the generated code
    "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
    # FP32 division must be the correctly rounded IEEE operation (quantizers)
    "-fhip-fp32-correctly-rounded-divide-sqrt",
    "-fno-fast-math",
    # MFMA results in VGPRs: the promotion FMAs read them without v_accvgpr_read
    # "-mllvm", "-amdgpu-mfma-vgpr-form",
    "-Wall",
    f"-I{os.path.join(ROOT, 'include')}",
]


def hipcc() -> str:
    for cand in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc"):
        if cand and os.path.exists(cand):
            return cand
    return "hipcc"


def build(asm_dir: str | None = None, verbose: bool = False) -> str:
    """Compile every HIP source into libfp8gemm.so.  Always recompiles."""
    tmp = LIB + ".tmp%d" % os.getpid()
    cmd = [hipcc(), *HIPCC_FLAGS, *SOURCES, "-o", tmp]
    if asm_dir:
        os.makedirs(asm_dir, exist_ok=True)
        cmd += ["-save-temps=obj"]
        cmd[cmd.index("-o") + 1] = os.path.join(asm_dir, "libfp8gemm.so")
    if verbose:
        print(" ".join(cmd), flush=True)
    res = subprocess.run(cmd, capture_output=True, text=True,
                         cwd=asm_dir if asm_dir else None)
    noise = "is not a recognized feature for this target"
    err = "\n".join(l for l in res.stderr.splitlines() if noise not in l and "(ignoring feature)" not in l)
    if res.returncode != 0:
        raise RuntimeError(f"hipcc failed ({res.returncode}):\n{err}")
    if err.strip() and verbose:
        print(err, file=sys.stderr)
    if asm_dir:
        return os.path.join(asm_dir, "libfp8gemm.so")
    os.replace(tmp, LIB)
    return LIB


if __name__ == "__main__":
    asm = None
    if "--asm" in sys.argv:
        asm = os.path.join(ROOT, "_build", "asm")
    print(build(asm_dir=asm, verbose=True))
