"""RMSNorm fused into the LoRA-SwiGLU MLP (lora_rmsnorm_swiglu_mlp_fwd/bwd)
against the oracle's composition of the two steps: rmsnorm_fwd then
mlp_fwd on the normalised rows, and mlp_bwd then rmsnorm_bwd for the raw
rows' gradient.  The GPU path folds the frozen norm weight into the gate/up
base weights (lora_fold_norm_weight) and never forms the normalised rows;
the oracle keeps W and w apart, as the layers define them."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import gen_config, gen_mlp

from gpu_helpers import check, dev, host, log

pytestmark = pytest.mark.gpu
EPS = 1e-5


def norm_weight(d, seed):
    # w ~ 1 + N(0, 0.1^2) in bf16, as the standalone RMSNorm tests draw it
    g = np.random.default_rng(seed)
    import torch
    w = (1.0 + 0.1 * g.standard_normal(d)).astype(np.float32)
    return torch.from_numpy(w).to(torch.bfloat16).float().numpy()


def run_fused(mi, w, x_scale=1.0, accumulate=False, rows=None, full_grads=True):
    import torch
    s = oracle.scaling(mi.alpha, mi.r)
    Xh = (mi.X * np.float32(x_scale)).astype(np.float32)
    Xh = torch.from_numpy(Xh).to(torch.bfloat16).float().numpy()   # raw rows, exact bf16
    X, dY, wd = dev(Xh, "bf16"), dev(mi.dY, "bf16"), dev(w, "bf16")
    Wd = {p: dev(mi.W[p], "bf16") for p in mi.W}
    Wf = {"gate": L.lora_fold_norm_weight(Wd["gate"], wd),
          "up": L.lora_fold_norm_weight(Wd["up"], wd), "down": Wd["down"]}
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    Y, e, g, rstd = L.lora_rmsnorm_swiglu_mlp_fwd(X, wd, EPS, Wf, A, B, mi.alpha)
    out = {}
    R = None
    if accumulate:
        R = np.random.default_rng(3).standard_normal((mi.T, mi.d)).astype(np.float32)
        R = torch.from_numpy(R).to(torch.bfloat16).float().numpy()
        out["dX"] = dev(R, "bf16")
    grads = L.lora_rmsnorm_swiglu_mlp_bwd(X, wd, rstd, Wf, A, B, mi.alpha, e, g, dY,
                                          accumulate_dx=accumulate, out=out)
    torch.cuda.synchronize()
    rows = np.arange(mi.T) if rows is None else rows
    rt = torch.from_numpy(rows).to("cuda")
    Xn, rr = oracle.rmsnorm_fwd(Xh[rows], w, EPS)
    assert np.allclose(host(rstd[rt]), rr, rtol=1e-5, atol=0), "rstd"
    Yr, er, gr = oracle.mlp_fwd(Xn, mi.W, mi.A, mi.B, s)
    check("Y", host(Y[rt]), Yr, "bf16")
    check("e", host(e[rt]), er, "bf16")
    check("g", host(g[rt]), gr, "bf16")
    dXn = oracle.mlp_bwd(Xn, mi.W, mi.A, mi.B, s, mi.dY[rows])["dX"]
    dXr = oracle.rmsnorm_bwd(Xh[rows], w, EPS, dXn)
    if accumulate:
        dXr = dXr + R[rows]
    check("dX (raw rows)", host(grads["dX"][rt]), dXr, "bf16")
    if full_grads:
        Xn_all, _ = oracle.rmsnorm_fwd(Xh, w, EPS)
        ref = oracle.mlp_bwd(Xn_all, mi.W, mi.A, mi.B, s, mi.dY, want_dx=False)
        for k, v in ref.items():
            if v is not None:
                check(k, host(grads[k]), v, "bf16")
    return grads


@pytest.mark.parametrize("T,d,f,r,bstd,xs", [
    (300, 320, 520, 16, 0.02, 1.0),     # ragged in every dimension, the dual rank-r pass
    (256, 256, 512, 8, 1.0, 1.0),       # LoRA-dominant adapters
    (200, 256, 768, 64, 0.5, 30.0),     # wide rank (separate rank-r passes), large activations
    (264, 192, 392, 32, 0.3, 1.0),      # the dual rank-r passes
    (37, 72, 40, 3, 0.5, 1.0),          # below one tile
], ids=lambda v: str(v))
def test_fused_norm_mlp(T, d, f, r, bstd, xs):
    log(f"fused norm + MLP T={T} d={d} f={f} r={r} b_std={bstd} x_scale={xs}")
    mi = gen_mlp(T, d, f, r, 16.0, "bf16", seed=T + d, b_std=bstd)
    run_fused(mi, norm_weight(d, seed=d), x_scale=xs)


def test_fused_norm_mlp_accumulates_residual_gradient():
    mi = gen_mlp(700, 512, 1024, 16, 16.0, "bf16", seed=12, b_std=0.3)
    run_fused(mi, norm_weight(512, seed=13), accumulate=True)


def test_fused_norm_mlp_T_zero():
    import torch
    mi = gen_mlp(4, 64, 128, 4, 16.0, "bf16", seed=2)
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    wd = dev(norm_weight(64, 1), "bf16")
    W = {p: dev(mi.W[p], "bf16") for p in mi.W}
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    Y, e, g, rstd = L.lora_rmsnorm_swiglu_mlp_fwd(X, wd, EPS, W, A, B, 16.0)
    o = {"dA_" + p: torch.full_like(A[p], 7.0) for p in A}
    o.update({"dB_" + p: torch.full_like(B[p], 7.0) for p in B})
    grads = L.lora_rmsnorm_swiglu_mlp_bwd(X, wd, rstd, W, A, B, 16.0, e, g, Y, out=o)
    torch.cuda.synchronize()
    for p in ("gate", "up", "down"):
        assert float(grads["dA_" + p].abs().max()) == 0.0
        assert float(grads["dB_" + p].abs().max()) == 0.0


def test_fused_norm_mlp_deterministic():
    import torch
    mi = gen_mlp(520, 384, 768, 16, 16.0, "bf16", seed=21)
    w = dev(norm_weight(384, 22), "bf16")
    X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
    Wd = {p: dev(mi.W[p], "bf16") for p in mi.W}
    Wf = {"gate": L.lora_fold_norm_weight(Wd["gate"], w), "up": L.lora_fold_norm_weight(Wd["up"], w),
          "down": Wd["down"]}
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    first = None
    for _ in range(4):
        Y, e, g, rstd = L.lora_rmsnorm_swiglu_mlp_fwd(X, w, EPS, Wf, A, B, 16.0)
        gr = L.lora_rmsnorm_swiglu_mlp_bwd(X, w, rstd, Wf, A, B, 16.0, e, g, dY)
        got = [Y, e, g, rstd] + [gr[k] for k in sorted(gr)]
        got = [t.clone() for t in got]
        if first is None:
            first = got
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, got))


def test_fold_norm_weight_bit_exact():
    import torch
    g = np.random.default_rng(4)
    W = torch.from_numpy(g.standard_normal((96, 200)).astype(np.float32) * 0.02).to(torch.bfloat16)
    w = torch.from_numpy(norm_weight(200, 5)).to(torch.bfloat16)
    got = L.lora_fold_norm_weight(W.cuda(), w.cuda()).cpu()
    # one fp32 product of two bf16 values, rounded once to bf16 (torch on the CPU)
    ref = (W.float() * w.float()[None, :]).to(torch.bfloat16)
    assert torch.equal(got.view(torch.int16), ref.view(torch.int16))
    Wc = W.cuda()
    L.lora_fold_norm_weight(Wc, w.cuda(), out=Wc)        # in place
    assert torch.equal(Wc.cpu().view(torch.int16), ref.view(torch.int16))


@pytest.mark.slow
def test_fused_norm_mlp_full_size():
    """Llama-3-8B MLP shapes (T = 8192, d = 4096, f = 14336, r = 16) with the
    norm in front: three whole 256-row tile bands and random rows of Y, e, g,
    dX; every adapter gradient in full."""
    mi = gen_config(3)
    T = mi.T
    r = np.random.default_rng(33)
    rows = np.unique(np.concatenate([np.arange(0, 256), np.arange(4096, 4352),
                                     np.arange(T - 256, T), r.integers(0, T, 40)]))
    log("fused norm + MLP at T=8192 d=4096 f=14336 r=16")
    run_fused(mi, norm_weight(mi.d, 34), rows=rows)


# ------------------------------------------------------------- q/k/v
def run_fused_qkv(T, k, nq, nkv, r, w, bstd=0.02, x_scale=1.0, accumulate=False, seed=1,
                  rows=None):
    """lora_rmsnorm_qkv_fwd/bwd against rmsnorm_fwd then linear_fwd per
    projection, and the projections' summed input gradient through
    rmsnorm_bwd; the GPU reads q/k/v weights folded with w."""
    import torch
    from lora_inputs import gen_linear
    q = gen_linear(T, k, nq, r, 16.0, "bf16", seed=seed, b_std=bstd)
    lis = {"q": q,
           "k": gen_linear(T, k, nkv, r, 16.0, "bf16", seed=seed + 1, b_std=bstd, X=q.X),
           "v": gen_linear(T, k, nkv, r, 16.0, "bf16", seed=seed + 2, b_std=bstd, X=q.X)}
    s = oracle.scaling(q.alpha, r)
    Xh = (q.X * np.float32(x_scale)).astype(np.float32)
    Xh = torch.from_numpy(Xh).to(torch.bfloat16).float().numpy()   # raw rows, exact bf16
    X, wd = dev(Xh, "bf16"), dev(w, "bf16")
    Wf = {p: L.lora_fold_norm_weight(dev(li.W, "bf16"), wd) for p, li in lis.items()}
    A = {p: dev(li.A, "bf16") for p, li in lis.items()}
    B = {p: dev(li.B, "bf16") for p, li in lis.items()}
    dY = {p: dev(li.dY, "bf16") for p, li in lis.items()}
    outs, rstd = L.lora_rmsnorm_qkv_fwd(X, wd, EPS, Wf, A, B, q.alpha)
    o = {}
    R = None
    if accumulate:
        R = np.random.default_rng(seed + 7).standard_normal((T, k)).astype(np.float32)
        R = torch.from_numpy(R).to(torch.bfloat16).float().numpy()
        o["dX"] = dev(R, "bf16")
    grads = L.lora_rmsnorm_qkv_bwd(X, wd, rstd, Wf, A, B, q.alpha, dY, accumulate_dx=accumulate,
                                   out=o)
    torch.cuda.synchronize()
    rows = np.arange(T) if rows is None else rows
    rt = torch.from_numpy(rows).to("cuda")
    Xn, rr = oracle.rmsnorm_fwd(Xh, w, EPS)
    assert np.allclose(host(rstd), rr, rtol=1e-5, atol=0), "rstd"
    dXn = 0.0
    for p, li in lis.items():
        check(p, host(outs[p][rt]), oracle.linear_fwd(Xn[rows], li.W, li.A, li.B, s), "bf16")
        dXp, dAr, dBr = oracle.linear_bwd(Xn, li.W, li.A, li.B, s, li.dY)
        check(f"dA_{p}", host(grads["dA_" + p]), dAr, "bf16")
        check(f"dB_{p}", host(grads["dB_" + p]), dBr, "bf16")
        dXn = dXn + dXp
    dXr = oracle.rmsnorm_bwd(Xh, w, EPS, dXn)
    if accumulate:
        dXr = dXr + R
    check("dX (raw rows)", host(grads["dX"][rt]), dXr[rows], "bf16")
    return outs, grads


@pytest.mark.parametrize("T,k,nq,nkv,r,bstd,xs", [
    (300, 320, 512, 256, 16, 0.02, 1.0),    # ragged tokens, k not a tile multiple
    (130, 256, 256, 256, 64, 0.02, 1.0),    # 3r = 192 side columns
    (200, 256, 512, 256, 8, 1.0, 30.0),     # LoRA-dominant adapters, large activations
    (37, 72, 256, 256, 3, 0.5, 1.0),        # below one tile
], ids=lambda v: str(v))
def test_fused_norm_qkv(T, k, nq, nkv, r, bstd, xs):
    log(f"fused norm + q/k/v T={T} k={k} nq={nq} nkv={nkv} r={r} b_std={bstd} x_scale={xs}")
    run_fused_qkv(T, k, nq, nkv, r, norm_weight(k, seed=k + 1), bstd=bstd, x_scale=xs, seed=T)


def test_fused_norm_qkv_accumulates_residual_gradient():
    log("fused norm + q/k/v, dX added to the residual stream's gradient")
    run_fused_qkv(260, 512, 512, 256, 16, norm_weight(512, seed=9), bstd=0.3, accumulate=True,
                  seed=8)


def test_fused_norm_qkv_T_zero():
    import torch
    k, nq, nkv, r = 64, 256, 256, 4
    X = torch.empty((0, k), dtype=torch.bfloat16, device="cuda")
    wd = dev(norm_weight(k, 1), "bf16")
    g = np.random.default_rng(3)
    W = {p: dev(g.standard_normal((n, k)) * 0.02, "bf16") for p, n in (("q", nq), ("k", nkv),
                                                                        ("v", nkv))}
    A = {p: dev(g.standard_normal((r, k)) * 0.1, "bf16") for p in "qkv"}
    B = {p: dev(g.standard_normal((W[p].shape[0], r)) * 0.1, "bf16") for p in "qkv"}
    outs, rstd = L.lora_rmsnorm_qkv_fwd(X, wd, EPS, W, A, B, 16.0)
    o = {"dA_" + p: torch.full_like(A[p], 7.0) for p in "qkv"}
    o.update({"dB_" + p: torch.full_like(B[p], 7.0) for p in "qkv"})
    grads = L.lora_rmsnorm_qkv_bwd(X, wd, rstd, W, A, B, 16.0, outs, out=o)
    torch.cuda.synchronize()
    for p in "qkv":
        assert float(grads["dA_" + p].abs().max()) == 0.0
        assert float(grads["dB_" + p].abs().max()) == 0.0


def test_fused_norm_qkv_deterministic():
    import torch
    first = None
    for _ in range(3):
        outs, grads = run_fused_qkv(520, 384, 512, 256, 16, norm_weight(384, seed=22), seed=21)
        got = [outs[p].clone() for p in "qkv"] + [grads[k].clone() for k in sorted(grads)]
        if first is None:
            first = got
        else:
            assert all(torch.equal(a, b) for a, b in zip(first, got))


@pytest.mark.slow
def test_fused_norm_qkv_full_size():
    """Llama-3-8B attention projections with the norm in front (T = 16384,
    k = 4096, nq = 4096, nkv = 1024, r = 64): three whole 256-row tile bands
    and random rows of Q, K, V and dX; every adapter gradient in full."""
    T = 16384
    g = np.random.default_rng(41)
    rows = np.unique(np.concatenate([np.arange(0, 256), np.arange(8192, 8448),
                                     np.arange(T - 256, T), g.integers(0, T, 40)]))
    log("fused norm + q/k/v at T=16384 k=4096 nq=4096 nkv=1024 r=64")
    run_fused_qkv(T, 4096, 4096, 1024, 64, norm_weight(4096, 42), seed=40, rows=rows)
