"""GPU parity at the benchmark workloads' full sizes, in the launch
configuration bench.py times (the same C-ABI calls on full tensors).

Outputs that are local to a token row (Y, e, g, dX) are checked on rows
that the oracle computes one by one: three whole 256-token tile bands (the
first, a seeded middle one and the last, which is the ragged one when T is
not a multiple of 256) over every column, plus seeded random rows; the
adapter gradients reduce over all tokens and are checked in full against
the float64 oracle.  Tolerance: 2e-2 relative Frobenius error per tensor
(bf16 storage, fp32 accumulation) and the element-wise bound of
gpu_helpers.check."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import gen_config

from gpu_helpers import check, dev, host, log, mlp_weights

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def sample_rows(T, n=40, seed=0, band=256):
    """Whole tile bands (first, a seeded middle one, last) plus n random rows."""
    r = np.random.default_rng(seed)
    nb = (T + band - 1) // band
    mid = int(r.integers(1, nb - 1)) if nb > 2 else 0
    bands = [np.arange(b * band, min(T, (b + 1) * band)) for b in sorted({0, mid, nb - 1})]
    rows = np.unique(np.concatenate(bands + [r.integers(0, T, n)]))
    return rows


def run_full_mlp(cfg, q4=None, minimal=False, transposed=False):
    import torch
    log(f"config {cfg} (4-bit form {q4}, minimal workspace {minimal}, caller-kept W^T "
        f"{transposed}): generating inputs")
    mi = gen_config(cfg, q4=q4)
    s = oracle.scaling(mi.alpha, mi.r)
    Wd, Wref = mlp_weights(mi)
    if transposed:
        Wd = {p: L.with_transpose(v) for p, v in Wd.items()}
    X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    log(f"config {cfg}: GPU fwd+bwd T={mi.T} d={mi.d} f={mi.f} r={mi.r}")
    Y, e, g = L.lora_swiglu_mlp_fwd(X, Wd, A, B, mi.alpha, minimal_workspace=minimal)
    grads = L.lora_swiglu_mlp_bwd(X, Wd, A, B, mi.alpha, e, g, dY, minimal_workspace=minimal)
    torch.cuda.synchronize()
    rows = sample_rows(mi.T, seed=cfg)
    rt = torch.from_numpy(rows).to("cuda")
    log(f"config {cfg}: oracle on {len(rows)} sampled rows")
    Yr, er, gr = oracle.mlp_fwd(mi.X[rows], Wref, mi.A, mi.B, s)
    check("Y[rows]", host(Y[rt]), Yr, "bf16")
    check("e[rows]", host(e[rt]), er, "bf16")
    check("g[rows]", host(g[rt]), gr, "bf16")
    dXr = oracle.mlp_bwd(mi.X[rows], Wref, mi.A, mi.B, s, mi.dY[rows])["dX"]
    check("dX[rows]", host(grads["dX"][rt]), dXr, "bf16")
    log(f"config {cfg}: oracle adapter gradients over all {mi.T} tokens")
    ref = oracle.mlp_bwd(mi.X, Wref, mi.A, mi.B, s, mi.dY, want_dx=False)
    for k, v in ref.items():
        if v is not None:
            check(k, host(grads[k]), v, "bf16")


@pytest.mark.parametrize("cfg", [2, 3, 5])
def test_full_mlp(cfg):
    run_full_mlp(cfg)


@pytest.mark.parametrize("cfg", [2, 3])
def test_full_mlp_transposed_weights(cfg):
    """The caller keeps W^T next to each frozen weight (the benchmark's
    default): both backward dX GEMMs run the K-contiguous form on it."""
    run_full_mlp(cfg, transposed=True)


def test_full_mlp_q4_minimal():
    """The 4-bit 8B MLP in the minimal workspace: every 4-bit GEMM decodes its
    codes inside the LDS fill (forward NT, backward NN with the K split
    between the gate and up weights)."""
    run_full_mlp(5, minimal=True)


@pytest.mark.parametrize("minimal", [False, True], ids=["fast", "minimal"])
def test_full_mlp_double_quantised(minimal):
    """The 4-bit 8B MLP with double-quantised block constants (minimal
    workspace: decoded inside the GEMMs)."""
    run_full_mlp(5, q4="dq", minimal=minimal)


def test_full_config4_attention_projections():
    """q/k/v share one input (their dX accumulate), o has its own, r = 64,
    T = 16384; every projection's outputs and gradients against the oracle."""
    import torch
    log("config 4: generating attention inputs")
    layers = gen_config(4, part="attn")["attn"]
    T = layers["q"].T
    rows = sample_rows(T, seed=4)
    rt = torch.from_numpy(rows).to("cuda")
    Xqkv = dev(layers["q"].X, "bf16")
    dX = torch.zeros_like(Xqkv)
    dX_ref = 0.0
    for i, name in enumerate(("q", "k", "v", "o")):
        li = layers[name]
        s = oracle.scaling(li.alpha, li.r)
        X = Xqkv if name != "o" else dev(li.X, "bf16")
        W, A, B, dY = (dev(v, "bf16") for v in (li.W, li.A, li.B, li.dY))
        log(f"config 4 {name}: T={T} k={li.k} n={li.n} r={li.r}")
        Y = L.lora_linear_fwd(X, W, A, B, li.alpha)
        if name == "o":
            dXo, dA, dB = L.lora_linear_bwd(X, W, A, B, li.alpha, dY)
        else:
            _, dA, dB = L.lora_linear_bwd(X, W, A, B, li.alpha, dY, dX=dX, accumulate_dx=i > 0)
        torch.cuda.synchronize()
        check(f"{name}.Y[rows]", host(Y[rt]), oracle.linear_fwd(li.X[rows], li.W, li.A, li.B, s), "bf16")
        _, dAr, dBr = oracle.linear_bwd(li.X, li.W, li.A, li.B, s, li.dY, want_dx=False)
        check(f"{name}.dA", host(dA), dAr, "bf16")
        check(f"{name}.dB", host(dB), dBr, "bf16")
        dXr = oracle.linear_bwd(li.X[rows], li.W, li.A, li.B, s, li.dY[rows])[0]
        if name == "o":
            check("o.dX[rows]", host(dXo[rt]), dXr, "bf16")
        else:
            dX_ref = dX_ref + dXr
    check("qkv.dX[rows] (sum of q, k, v)", host(dX[rt]), dX_ref, "bf16")


def test_full_config4_mlp():
    """The MLP of the 8B-attention-plus-MLP workload: T = 16384, r = 64."""
    import torch
    mi = gen_config(4, part="mlp")["mlp"]
    s = oracle.scaling(mi.alpha, mi.r)
    Wd = {p: dev(mi.W[p], "bf16") for p in mi.W}
    X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    log(f"config 4 mlp: T={mi.T} d={mi.d} f={mi.f} r={mi.r}")
    Y, e, g = L.lora_swiglu_mlp_fwd(X, Wd, A, B, mi.alpha)
    grads = L.lora_swiglu_mlp_bwd(X, Wd, A, B, mi.alpha, e, g, dY)
    torch.cuda.synchronize()
    rows = sample_rows(mi.T, seed=44)
    rt = torch.from_numpy(rows).to("cuda")
    Yr, er, gr = oracle.mlp_fwd(mi.X[rows], mi.W, mi.A, mi.B, s)
    check("Y[rows]", host(Y[rt]), Yr, "bf16")
    check("e[rows]", host(e[rt]), er, "bf16")
    dXr = oracle.mlp_bwd(mi.X[rows], mi.W, mi.A, mi.B, s, mi.dY[rows])["dX"]
    check("dX[rows]", host(grads["dX"][rt]), dXr, "bf16")
    log("config 4 mlp: oracle adapter gradients over all tokens")
    ref = oracle.mlp_bwd(mi.X, mi.W, mi.A, mi.B, s, mi.dY, want_dx=False)
    for k, v in ref.items():
        if v is not None:
            check(k, host(grads[k]), v, "bf16")


def test_full_dequant4_8b_weight():
    """Standalone decode of one 8B-MLP 4-bit weight [14336 x 4096], bit-exact."""
    import torch
    mi = gen_config(5)
    q = mi.q4["gate"]
    out = L.lora_dequant4(L.to_device_q4(q))
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.decode_q4_bits(q.codes, q.absmax, q.codebook, q.n, q.k)
    assert np.array_equal(got, ref)


def test_full_decode_dq_8b_weight():
    """Decode of one 8B-MLP weight [14336 x 4096] with double-quantised
    block constants, bit-exact."""
    import torch
    mi = gen_config(5, q4="dq")
    q = mi.q4["down"]
    out = L.lora_decode_weight(L.to_device_q4(q))
    torch.cuda.synchronize()
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.decode_q4dq_bits(q.codes, q.absmax_codes, q.absmax_codebook, q.absmax_scale,
                                  q.absmax_offset, q.codebook, q.n, q.k)
    assert np.array_equal(got, ref)


def test_full_config4_fused_qkv():
    """The fused q/k/v path at the 8B attention shape (T = 16384, d = 4096,
    d_kv = 1024, r = 64): sampled rows of q, k, v and dX, full adapter
    gradients."""
    import torch
    log("config 4: generating attention inputs (fused q/k/v)")
    layers = gen_config(4, part="attn")["attn"]
    T = layers["q"].T
    rows = sample_rows(T, seed=41)
    rt = torch.from_numpy(rows).to("cuda")
    X = dev(layers["q"].X, "bf16")
    W = {p: dev(layers[p].W, "bf16") for p in ("q", "k", "v")}
    A = {p: dev(layers[p].A, "bf16") for p in ("q", "k", "v")}
    B = {p: dev(layers[p].B, "bf16") for p in ("q", "k", "v")}
    dY = {p: dev(layers[p].dY, "bf16") for p in ("q", "k", "v")}
    alpha = layers["q"].alpha
    out = L.lora_qkv_fwd(X, W, A, B, alpha)
    g = L.lora_qkv_bwd(X, W, A, B, alpha, dY)
    torch.cuda.synchronize()
    dX_ref = 0.0
    for p in ("q", "k", "v"):
        li = layers[p]
        s = oracle.scaling(li.alpha, li.r)
        check(f"{p}[rows]", host(out[p][rt]), oracle.linear_fwd(li.X[rows], li.W, li.A, li.B, s),
              "bf16")
        _, dAr, dBr = oracle.linear_bwd(li.X, li.W, li.A, li.B, s, li.dY, want_dx=False)
        check(f"dA_{p}", host(g["dA_" + p]), dAr, "bf16")
        check(f"dB_{p}", host(g["dB_" + p]), dBr, "bf16")
        dX_ref = dX_ref + oracle.linear_bwd(li.X[rows], li.W, li.A, li.B, s, li.dY[rows])[0]
    check("dX[rows]", host(g["dX"][rt]), dX_ref, "bf16")


def test_full_rmsnorm_8b_rows():
    """RMSNorm forward and backward over T=8192 rows of d=4096 (the 8B
    model's hidden size), every element against the oracle."""
    import torch
    from lora_inputs import gen_rmsnorm
    ri = gen_rmsnorm(8192, 4096, "bf16", seed=77)
    X, w, dY = dev(ri.X, "bf16"), dev(ri.w, "bf16"), dev(ri.dY, "bf16")
    Y, rstd = L.lora_rmsnorm_fwd(X, w, ri.eps)
    dX = L.lora_rmsnorm_bwd(X, w, rstd, dY)
    torch.cuda.synchronize()
    Yr, rr = oracle.rmsnorm_fwd(ri.X, ri.w, ri.eps)
    assert np.allclose(host(rstd), rr, rtol=1e-5, atol=0)
    check("Y", host(Y), Yr, "bf16")
    check("dX", host(dX), oracle.rmsnorm_bwd(ri.X, ri.w, ri.eps, ri.dY), "bf16")
