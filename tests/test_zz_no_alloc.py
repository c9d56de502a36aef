"""lora_linear_bwd_noalloc (the allocation-free linear backward, scratch in
a static per-GPU device array) against lora_linear_bwd with the minimal
workspace: the same kernels over the same inputs, so every output must match
bit for bit.  Two calls in a row, the second with smaller inputs (the array
keeps the first call's contents), in bf16 (dense and 4-bit) and fp32, and
the over-size refusal."""
import ctypes

import numpy as np
import pytest

import lora_linear_fwd_amd as L
from lora_inputs import gen_linear

from gpu_helpers import dev, linear_weight, log

pytestmark = pytest.mark.gpu


def _pair(li, accumulate=False):
    import torch
    W, _ = linear_weight(li)
    X, A, B, dY = (dev(v, li.dtype) for v in (li.X, li.A, li.B, li.dY))
    torch.manual_seed(5)
    dX0 = torch.randn((li.T, li.k), device="cuda").to(X.dtype)
    # reference: the existing entry point with the minimal workspace
    ref_dX = dX0.clone()
    ref_dA, ref_dB = torch.empty_like(A), torch.empty_like(B)
    L.lora_linear_bwd(X, W, A, B, li.alpha, dY, dX=ref_dX, accumulate_dx=accumulate, dA=ref_dA,
                      dB=ref_dB, minimal_workspace=True)
    dX = dX0.clone()
    dA, dB = torch.full_like(A, float("nan")), torch.full_like(B, float("nan"))
    L.lora_linear_bwd_noalloc(X, W, A, B, li.alpha, dY, dX, dA, dB, accumulate_dx=accumulate)
    torch.cuda.synchronize()
    for name, got, ref in (("dX", dX, ref_dX), ("dA", dA, ref_dA), ("dB", dB, ref_dB)):
        same = torch.equal(got.view(torch.int16) if got.dtype == torch.bfloat16 else got.view(torch.int32),
                           ref.view(torch.int16) if ref.dtype == torch.bfloat16 else ref.view(torch.int32))
        log(f"  {name}: bit-identical {same}")
        assert same, f"{name} differs from lora_linear_bwd"


@pytest.mark.parametrize("dtype,q4", [("bf16", False), ("bf16", True), ("f32", False)])
def test_noalloc_matches_workspace_call_twice(dtype, q4):
    big = gen_linear(1000, 512, 768, 16, 16.0, dtype, seed=61, q4=q4)
    small = gen_linear(77, 256, 320, 8, 16.0, dtype, seed=62, q4=q4)
    log(f"no-alloc {dtype} q4={q4}: T=1000 k=512 n=768 r=16, then T=77 k=256 n=320 r=8")
    _pair(big)
    _pair(small, accumulate=True)


def test_noalloc_refuses_oversize():
    import torch
    T, k, n, r = 65536, 4096, 4096, 128
    need = L.workspace_bytes(L.OP_LINEAR_BWD | L.LORA_WS_MINIMAL, L.LORA_BF16, 0, T, k, n, r)
    assert need > L.LORA_NOALLOC_SCRATCH_BYTES
    p = ctypes.c_void_p(1 << 20)
    wst = L.LoraWeightC(L.LORA_W_DENSE, 0, p.value, None, None, None)
    st = L.lib().lora_linear_bwd_noalloc(L.LORA_BF16, T, k, n, r, 16.0, p, ctypes.byref(wst), p,
                                         p, p, p, p, p, 0, None)
    assert st == 4   # LORA_ERR_WORKSPACE, before any launch
    torch.cuda.synchronize()
