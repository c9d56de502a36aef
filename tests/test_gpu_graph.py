"""The entry points under HIP graph capture: one LoRA-SwiGLU MLP forward +
backward step (and a q/k/v step) captured on a side stream and replayed
several times, with eager work and synchronisations between the replays.
The library issues no allocation, memset or synchronisation of its own, so
every replay must reproduce the eager results bit for bit (the kernels'
reductions run in a fixed order)."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
from lora_inputs import gen_linear, gen_mlp

from gpu_helpers import dev, log, mlp_weights

pytestmark = pytest.mark.gpu


def _bits(t):
    import torch
    return t.view(torch.int16).cpu().numpy().copy()


@pytest.mark.parametrize("form", [False, "dq"], ids=["bf16", "q4dq"])
@pytest.mark.parametrize("ws", ["fast", "minimal"])
def test_mlp_step_graph_replays_match_eager(form, ws):
    import torch
    log(f"graph: mlp form={form} ws={ws}")
    T, d, f, r = 300, 256, 576, 16
    mi = gen_mlp(T, d, f, r, 16.0, "bf16", seed=51, q4=form)
    Wd, _ = mlp_weights(mi)
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
    wfmt = L._wfmt(Wd["gate"])
    flag = L.LORA_WS_MINIMAL if ws == "minimal" else 0
    # one buffer, a view of exactly each call's strategy size (the size
    # handed to the library selects the strategy)
    nf = L.workspace_bytes(L.OP_MLP_FWD | flag, L.LORA_BF16, wfmt, T, d, f, r)
    nb = L.workspace_bytes(L.OP_MLP_BWD | flag, L.LORA_BF16, wfmt, T, d, f, r)
    wsb = torch.empty(max(nf, nb), dtype=torch.uint8, device="cuda")
    wsf, wsbw = wsb[:nf], wsb[:nb]
    Y = torch.empty((T, d), dtype=torch.bfloat16, device="cuda")
    e = torch.empty((T, f), dtype=torch.bfloat16, device="cuda")
    g = torch.empty((T, f), dtype=torch.bfloat16, device="cuda")
    out = {"dX": torch.empty((T, d), dtype=torch.bfloat16, device="cuda")}
    for p in ("gate", "up", "down"):
        out["dA_" + p] = torch.empty_like(A[p])
        out["dB_" + p] = torch.empty_like(B[p])

    def step(stream):
        L.lora_swiglu_mlp_fwd(X, Wd, A, B, mi.alpha, Y=Y, e=e, g=g, workspace=wsf, stream=stream)
        L.lora_swiglu_mlp_bwd(X, Wd, A, B, mi.alpha, e, g, dY, out=out, workspace=wsbw,
                              stream=stream)

    outs = lambda: [Y, e, g] + [out[k] for k in sorted(out)]
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [_bits(t) for t in outs()]

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs():
            t.fill_(7.0)              # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(outs()):
            assert np.array_equal(_bits(t), ref[i]), f"replay {rep}, output {i}"


def test_qkv_step_graph_replays_match_eager():
    import torch
    log("graph: qkv")
    T, k, nq, nkv, r = 130, 256, 512, 256, 16
    lis = {p: gen_linear(T, k, n, r, 16.0, "bf16", seed=60 + i)
           for i, (p, n) in enumerate((("q", nq), ("k", nkv), ("v", nkv)))}
    X = dev(lis["q"].X, "bf16")
    W = {p: dev(li.W, "bf16") for p, li in lis.items()}
    A = {p: dev(li.A, "bf16") for p, li in lis.items()}
    B = {p: dev(li.B, "bf16") for p, li in lis.items()}
    dY = {p: dev(li.dY, "bf16") for p, li in lis.items()}
    nbytes = max(int(L.lib().lora_qkv_workspace_bytes(op, L.LORA_BF16, 0, T, k, nq, nkv, r))
                 for op in (L.OP_QKV_FWD, L.OP_QKV_BWD))
    wsb = torch.empty(nbytes, dtype=torch.uint8, device="cuda")
    o = L.lora_qkv_fwd(X, W, A, B, 16.0, workspace=wsb)
    gr = L.lora_qkv_bwd(X, W, A, B, 16.0, dY, workspace=wsb)
    torch.cuda.synchronize()
    tensors = [o[p] for p in ("q", "k", "v")] + [gr[kk] for kk in sorted(gr)]
    ref = [_bits(t) for t in tensors]

    def step(stream):
        L.lora_qkv_fwd(X, W, A, B, 16.0, out=o, workspace=wsb, stream=stream)
        L.lora_qkv_bwd(X, W, A, B, 16.0, dY, dX=gr["dX"], out=gr, workspace=wsb, stream=stream)

    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in tensors:
            t.fill_(3.0)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(tensors):
            assert np.array_equal(_bits(t), ref[i]), f"replay {rep}, tensor {i}"


@pytest.mark.parametrize("part", ["mlp", "qkv"])
def test_norm_fused_step_graph_replays_match_eager(part):
    """The norm-fused MLP and q/k/v steps (rstd-only norm pass, row-scaled
    epilogues, the norm coefficient and the raw rows' gradient) under graph
    capture, residual-gradient accumulation included."""
    import torch
    log(f"graph: norm-fused {part}")
    g = np.random.default_rng(71)
    if part == "mlp":
        T, d, f, r = 300, 256, 576, 16
        mi = gen_mlp(T, d, f, r, 16.0, "bf16", seed=72)
        Wd, _ = mlp_weights(mi)
        w = dev(1.0 + 0.1 * g.standard_normal(d), "bf16")
        W = dict(Wd, gate=L.lora_fold_norm_weight(Wd["gate"], w),
                 up=L.lora_fold_norm_weight(Wd["up"], w))
        A = {p: dev(mi.A[p], "bf16") for p in mi.A}
        B = {p: dev(mi.B[p], "bf16") for p in mi.B}
        X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
        nb = max(L.workspace_bytes(op, L.LORA_BF16, 0, T, d, f, r)
                 for op in (L.OP_RMSNORM_MLP_FWD, L.OP_RMSNORM_MLP_BWD))
        wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")
        Y, e, gg, rstd = L.lora_rmsnorm_swiglu_mlp_fwd(X, w, 1e-5, W, A, B, 16.0, workspace=wsb)
        R = dev(g.standard_normal((T, d)), "bf16")
        out = {"dX": torch.empty_like(X)}
        for p in ("gate", "up", "down"):
            out["dA_" + p] = torch.empty_like(A[p])
            out["dB_" + p] = torch.empty_like(B[p])

        def step(stream):
            out["dX"].copy_(R)     # the residual branch's gradient, accumulated into
            L.lora_rmsnorm_swiglu_mlp_fwd(X, w, 1e-5, W, A, B, 16.0, Y=Y, e=e, g=gg, rstd=rstd,
                                          workspace=wsb, stream=stream)
            L.lora_rmsnorm_swiglu_mlp_bwd(X, w, rstd, W, A, B, 16.0, e, gg, dY,
                                          accumulate_dx=True, out=out, workspace=wsb,
                                          stream=stream)
        outs = lambda: [Y, e, gg, rstd] + [out[k] for k in sorted(out)]
    else:
        T, k, nq, nkv, r = 130, 256, 512, 256, 16
        lis = {p: gen_linear(T, k, n, r, 16.0, "bf16", seed=80 + i)
               for i, (p, n) in enumerate((("q", nq), ("k", nkv), ("v", nkv)))}
        X = dev(lis["q"].X, "bf16")
        w = dev(1.0 + 0.1 * g.standard_normal(k), "bf16")
        W = {p: L.lora_fold_norm_weight(dev(li.W, "bf16"), w) for p, li in lis.items()}
        A = {p: dev(li.A, "bf16") for p, li in lis.items()}
        B = {p: dev(li.B, "bf16") for p, li in lis.items()}
        dY = {p: dev(li.dY, "bf16") for p, li in lis.items()}
        nb = max(int(L.lib().lora_qkv_workspace_bytes(op, L.LORA_BF16, 0, T, k, nq, nkv, r))
                 for op in (L.OP_RMSNORM_QKV_FWD, L.OP_RMSNORM_QKV_BWD))
        wsb = torch.empty(nb, dtype=torch.uint8, device="cuda")
        o, rstd = L.lora_rmsnorm_qkv_fwd(X, w, 1e-5, W, A, B, 16.0, workspace=wsb)
        gr = L.lora_rmsnorm_qkv_bwd(X, w, rstd, W, A, B, 16.0, dY, workspace=wsb)

        def step(stream):
            L.lora_rmsnorm_qkv_fwd(X, w, 1e-5, W, A, B, 16.0, out=o, rstd=rstd, workspace=wsb,
                                   stream=stream)
            L.lora_rmsnorm_qkv_bwd(X, w, rstd, W, A, B, 16.0, dY, out=gr, workspace=wsb,
                                   stream=stream)
        outs = lambda: [o[p] for p in ("q", "k", "v")] + [rstd] + [gr[kk] for kk in sorted(gr)]

    bits = lambda t: t.view(torch.int16 if t.dtype == torch.bfloat16 else torch.int32).cpu().numpy()
    step(torch.cuda.current_stream())
    torch.cuda.synchronize()
    ref = [bits(t).copy() for t in outs()]
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    graph = torch.cuda.CUDAGraph()
    with torch.cuda.stream(side):
        with torch.cuda.graph(graph, stream=side):
            step(side)
    torch.cuda.synchronize()
    for rep in range(3):
        for t in outs():
            t.fill_(5.0)              # eager work between replays
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        for i, t in enumerate(outs()):
            assert np.array_equal(bits(t), ref[i]), f"replay {rep}, output {i}"
