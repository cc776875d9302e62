"""The Python binding refuses output buffers that do not match what the
kernels write (shape, type, layout, device) before anything is launched, so a
wrong buffer raises instead of being written past its end."""
import numpy as np
import pytest
import torch

import fine_grained_block_e4m3_amd as fp8
import oracle
import workloads
from gpu_helpers import dev, say

pytestmark = pytest.mark.gpu


def _operands(M=64, N=256, K=256):
    wl = workloads.dense(M, N, K, seed=3)
    xq, sa = oracle.quant_1x128(wl.x)
    wq, sb = oracle.quant_128x128(wl.w)
    return wl, [dev(t) for t in (xq, sa, wq, sb)]


def _untouched(t: torch.Tensor, fill) -> bool:
    torch.cuda.synchronize()
    return bool((t == fill).all().item())


def test_gemm_refuses_wrong_out():
    _, a = _operands()
    say("binding: gemm_nt out checks")
    for bad, err in [(torch.full((64, 255), 7, dtype=torch.bfloat16, device="cuda"), ValueError),
                     (torch.full((63, 256), 7, dtype=torch.bfloat16, device="cuda"), ValueError),
                     (torch.full((64, 256), 7, dtype=torch.float16, device="cuda"), TypeError),
                     (torch.full((256, 64), 7, dtype=torch.bfloat16, device="cuda").t(), ValueError),
                     (torch.full((64, 256), 7, dtype=torch.bfloat16), ValueError)]:
        with pytest.raises(err):
            fp8.gemm_nt(*a, out=bad)
        if bad.is_cuda:
            assert _untouched(bad, 7)
    ok = torch.empty((64, 256), dtype=torch.bfloat16, device="cuda")
    assert fp8.gemm_nt(*a, out=ok) is ok


def test_quantizers_refuse_wrong_out():
    wl, _ = _operands()
    x, w = dev(wl.x), dev(wl.w)
    say("binding: quantizer out checks")
    xq = torch.full((64, 256), 7, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fp8.quant_1x128(x, out=(xq, torch.empty((2, 63), dtype=torch.float32, device="cuda")))
    with pytest.raises(TypeError):
        fp8.quant_1x128(x, out=(xq, torch.empty((2, 64), dtype=torch.float64, device="cuda")))
    assert _untouched(xq, 7)
    wq = torch.full((256, 256), 7, dtype=torch.uint8, device="cuda")
    with pytest.raises(ValueError):
        fp8.quant_128x128(w, out=(wq, torch.empty((2, 3), dtype=torch.float32, device="cuda")))
    assert _untouched(wq, 7)
    with pytest.raises(ValueError):
        fp8.quant_mx(x, out=(torch.empty((64, 128), dtype=torch.uint8, device="cuda"),
                             torch.empty((2, 64), dtype=torch.int32, device="cuda")))
    with pytest.raises(ValueError):
        fp8.quant_mxfp4(w, out=(torch.empty((256, 256), dtype=torch.uint8, device="cuda"),
                                torch.empty((2, 256), dtype=torch.int32, device="cuda")))


def test_grouped_refuse_wrong_out():
    E, max_m, N, K = 2, 64, 256, 256
    wl = workloads.masked(E, max_m, N, K, seed=9)
    xq, sa = oracle.quant_1x128(wl.x, oracle.FLAG_UE8M0)
    wq, sb = oracle.quant_128x128(wl.w, oracle.FLAG_UE8M0)
    a = [dev(xq.reshape(E, max_m, K)), dev(sa), dev(wq.reshape(E, N, K)),
         dev(sb.reshape(E, N // 128, K // 128)), dev(np.asarray(wl.masked_m, np.int32))]
    say("binding: masked out checks")
    flat = torch.full((E * max_m, N), 7, dtype=torch.bfloat16, device="cuda")
    with pytest.raises(ValueError):
        fp8.grouped_gemm_masked(*a, ue8m0=True, out=flat)
    assert _untouched(flat, 7)
    idx = dev(np.zeros(E * max_m, np.int32))
    with pytest.raises(ValueError):
        fp8.grouped_gemm_contiguous(a[0].reshape(E * max_m, K), a[1], a[2], a[3], idx,
                                    out=torch.empty((E * max_m, N + 1), dtype=torch.bfloat16,
                                                    device="cuda"))
