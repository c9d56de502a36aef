"""GPU parity of the fused q/k/v LoRA projections (lora_qkv_fwd / _bwd)
against the float64 oracle applied to each projection: the fused GEMM path
(bf16, nq and nkv multiples of 256, 3r <= 256), whose backward dX GEMM reads
dQ, dK, dV and the three W^T (the caller's, or transposed per call) as three
K sources where the widths are multiples of 64 and a packed [dQ | dK | dV]
otherwise, and the per-projection paths (other shapes, large r, fp32,
minimal workspace)."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import gen_linear

from gpu_helpers import check, dev, host, linear_weight, log

pytestmark = pytest.mark.gpu


def make_qkv(T, k, nq, nkv, r, dtype="bf16", seed=1, b_std=0.02, q4=False):
    q = gen_linear(T, k, nq, r, 16.0, dtype, seed=seed, b_std=b_std, q4=q4)
    kk = gen_linear(T, k, nkv, r, 16.0, dtype, seed=seed + 1, b_std=b_std, q4=q4, X=q.X)
    v = gen_linear(T, k, nkv, r, 16.0, dtype, seed=seed + 2, b_std=b_std, q4=q4, X=q.X)
    return {"q": q, "k": kk, "v": v}


def run_and_check(lis, ws="fast", accumulate=False):
    import torch
    li0 = lis["q"]
    dt = li0.dtype
    s = oracle.scaling(li0.alpha, li0.r)
    X = dev(li0.X, dt)
    W, Wref, A, B, dY = {}, {}, {}, {}, {}
    for p, li in lis.items():
        W[p], Wref[p] = linear_weight(li)
        A[p], B[p], dY[p] = dev(li.A, dt), dev(li.B, dt), dev(li.dY, dt)
    mw = ws == "minimal"
    if ws == "wt":   # caller-kept transposes next to the dense weights
        W = {p: L.with_transpose(w) for p, w in W.items()}
    out = L.lora_qkv_fwd(X, W, A, B, li0.alpha, minimal_workspace=mw)
    dX0 = None
    if accumulate:
        dX0 = np.random.default_rng(5).standard_normal(li0.X.shape).astype(np.float32)
        dX = dev(dX0, dt)
        dX0 = host(dX)
    else:
        dX = None
    g = L.lora_qkv_bwd(X, W, A, B, li0.alpha, dY, dX=dX, accumulate_dx=accumulate,
                       minimal_workspace=mw)
    torch.cuda.synchronize()
    dX_ref = 0.0 if dX0 is None else dX0
    for p, li in lis.items():
        check(f"{p}", host(out[p]), oracle.linear_fwd(li.X, Wref[p], li.A, li.B, s), dt)
        dXr, dAr, dBr = oracle.linear_bwd(li.X, Wref[p], li.A, li.B, s, li.dY)
        check(f"dA_{p}", host(g["dA_" + p]), dAr, dt)
        check(f"dB_{p}", host(g["dB_" + p]), dBr, dt)
        dX_ref = dX_ref + dXr
    check("dX", host(g["dX"]), dX_ref, dt)


@pytest.mark.parametrize("ws", ["fast", "minimal", "wt"])
@pytest.mark.parametrize("shape", [(300, 320, 512, 256, 16), (130, 256, 256, 256, 64),
                                   (37, 72, 264, 136, 3), (70, 128, 256, 256, 100)],
                         ids=lambda s: "x".join(map(str, s)))
def test_qkv_bf16(shape, ws):
    T, k, nq, nkv, r = shape
    log(f"qkv bf16 T={T} k={k} nq={nq} nkv={nkv} r={r} ws={ws}")
    run_and_check(make_qkv(T, k, nq, nkv, r, seed=T + r), ws=ws)


def test_qkv_lora_dominant():
    log("qkv bf16 lora-dominant")
    run_and_check(make_qkv(300, 320, 512, 256, 16, seed=3, b_std=1.0))


def test_qkv_accumulate_dx():
    log("qkv bf16 accumulate dX")
    run_and_check(make_qkv(200, 256, 256, 256, 16, seed=4, b_std=0.5), accumulate=True)


@pytest.mark.parametrize("ws", ["fast", "minimal"])
def test_qkv_q4(ws):
    log(f"qkv q4 ws={ws}")
    run_and_check(make_qkv(130, 256, 512, 256, 16, seed=6, q4=True), ws=ws)


def test_qkv_fp32():
    log("qkv fp32")
    run_and_check(make_qkv(37, 48, 40, 24, 5, dtype="f32", seed=8))
