"""GPU parity of the RMSNorm step in front of the projections
(lora_rmsnorm_fwd / _bwd) against the float64 oracle, alone and chained with
the LoRA-SwiGLU MLP as a decoder layer's MLP half: xn = rmsnorm(X), Y =
mlp(xn), and the backward into the residual stream.  Tolerances: each bf16
output is one rounding of an fp32 evaluation, so besides the 2e-2 relative
Frobenius bound every element must lie within 2^-7 of its magnitude (plus a
floor for values near zero); rstd within 1e-5 relative; fp32 within 1e-4."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import gen_mlp, gen_rmsnorm

from gpu_helpers import check, dev, host, log, mlp_weights

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


def _elementwise(name, got, ref, floor):
    bound = 2.0 ** -7 * np.abs(ref) + floor
    worst = float(np.max(np.abs(got - ref) / bound)) if ref.size else 0.0
    log(f"  {name}: worst |err| / bound = {worst:.3f}")
    assert worst <= 1.0, name


def run_norm(ri, accumulate=False):
    import torch
    X, w, dY = dev(ri.X, ri.dtype), dev(ri.w, ri.dtype), dev(ri.dY, ri.dtype)
    Y, rstd = L.lora_rmsnorm_fwd(X, w, ri.eps)
    dX0 = None
    if accumulate:
        dX = dev(np.random.default_rng(2).standard_normal(ri.X.shape).astype(np.float32), ri.dtype)
        dX0 = host(dX)
        L.lora_rmsnorm_bwd(X, w, rstd, dY, dX=dX, accumulate=True)
    else:
        dX = L.lora_rmsnorm_bwd(X, w, rstd, dY)
    _sync()
    return host(Y), host(rstd), host(dX), dX0


def check_norm(ri, accumulate=False):
    Y, rstd, dX, dX0 = run_norm(ri, accumulate)
    Yr, rr = oracle.rmsnorm_fwd(ri.X, ri.w, ri.eps)
    dXr = oracle.rmsnorm_bwd(ri.X, ri.w, ri.eps, ri.dY)
    if dX0 is not None:
        dXr = dXr + dX0
    assert np.allclose(rstd, rr, rtol=1e-5, atol=0), np.max(np.abs(rstd / rr - 1))
    check("Y", Y, Yr, ri.dtype)
    check("dX", dX, dXr, ri.dtype)
    if ri.dtype == "bf16":
        _elementwise("Y", Y, Yr, 2.0 ** -7 * 1e-3)
        # dX is a difference of two terms; the floor covers their fp32 cancellation
        scale = np.max(np.abs(dXr), axis=1, keepdims=True)
        _elementwise("dX", dX, dXr, 2.0 ** -7 * 1e-3 * scale)


NORM_SHAPES = [(300, 4096), (37, 72), (1, 8), (513, 136), (260, 5120)]


@pytest.mark.parametrize("shape", NORM_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_rmsnorm_bf16(shape):
    T, d = shape
    log(f"rmsnorm bf16 T={T} d={d}")
    check_norm(gen_rmsnorm(T, d, "bf16", seed=T + d))


def test_rmsnorm_bf16_accumulate_into_residual_grad():
    log("rmsnorm bf16 accumulate")
    check_norm(gen_rmsnorm(130, 1024, "bf16", seed=5), accumulate=True)


def test_rmsnorm_large_activations():
    # residual streams grow with depth: rows of magnitude ~50
    check_norm(gen_rmsnorm(64, 2048, "bf16", seed=6, x_std=50.0))


@pytest.mark.parametrize("shape", [(67, 50), (5, 4096)], ids=lambda s: "x".join(map(str, s)))
def test_rmsnorm_fp32(shape):
    T, d = shape
    log(f"rmsnorm fp32 T={T} d={d}")
    check_norm(gen_rmsnorm(T, d, "f32", seed=T * d))
    check_norm(gen_rmsnorm(T, d, "f32", seed=T * d + 1), accumulate=True)


def test_rmsnorm_deterministic():
    ri = gen_rmsnorm(257, 4096, "bf16", seed=8)
    a, b = run_norm(ri), run_norm(ri)
    for x, y in zip(a[:3], b[:3]):
        assert np.array_equal(x, y)


def test_rmsnorm_T_zero():
    import torch
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    w = torch.ones(64, dtype=torch.bfloat16, device="cuda")
    Y, rstd = L.lora_rmsnorm_fwd(X, w, 1e-5)
    dX = L.lora_rmsnorm_bwd(X, w, rstd, X)
    _sync()
    assert Y.shape == (0, 64) and dX.shape == (0, 64)


@pytest.mark.parametrize("ws", ["fast", "minimal"])
def test_rmsnorm_then_mlp_layer(ws):
    """xn = rmsnorm(X); Y = mlp(xn); backward into the residual stream:
    dX_res = dY_res + rmsnorm_bwd(mlp_bwd(dY_res)) (the residual add keeps
    the layer output's gradient)."""
    T, d, f, r = 300, 256, 520, 16
    log(f"rmsnorm + mlp T={T} d={d} f={f} r={r} ws={ws}")
    ri = gen_rmsnorm(T, d, "bf16", seed=41)
    mi = gen_mlp(T, d, f, r, 16.0, "bf16", seed=42)
    s = oracle.scaling(mi.alpha, mi.r)
    Wd, Wref = mlp_weights(mi)
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    X, w, dYres = dev(ri.X, "bf16"), dev(ri.w, "bf16"), dev(mi.dY, "bf16")
    mw = ws == "minimal"
    xn, rstd = L.lora_rmsnorm_fwd(X, w, ri.eps)
    Y, e, g = L.lora_swiglu_mlp_fwd(xn, Wd, A, B, mi.alpha, minimal_workspace=mw)
    grads = L.lora_swiglu_mlp_bwd(xn, Wd, A, B, mi.alpha, e, g, dYres, minimal_workspace=mw)
    dX = dYres.clone()
    L.lora_rmsnorm_bwd(X, w, rstd, grads["dX"], dX=dX, accumulate=True)
    _sync()
    xr, _ = oracle.rmsnorm_fwd(ri.X, ri.w, ri.eps)
    Yr, _, _ = oracle.mlp_fwd(xr, Wref, mi.A, mi.B, s)
    ref = oracle.mlp_bwd(xr, Wref, mi.A, mi.B, s, mi.dY)
    dXr = mi.dY + oracle.rmsnorm_bwd(ri.X, ri.w, ri.eps, ref["dX"])
    check("Y", host(Y), Yr, "bf16")
    check("dX (residual stream)", host(dX), dXr, "bf16")
    for p in ("gate", "up", "down"):
        check("dA_" + p, host(grads["dA_" + p]), ref["dA_" + p], "bf16")
        check("dB_" + p, host(grads["dB_" + p]), ref["dB_" + p], "bf16")
