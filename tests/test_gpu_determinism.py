"""Bitwise reproducibility of the LoRA-SwiGLU MLP step at full size.

Every reduction in the library runs in a fixed order, so repeated forward +
backward calls on the same inputs must give identical bits.  A race in a
GEMM pipeline (a stage refilled while another wave still reads it) shows up
here as rare differences that a tolerance-based parity check can miss, so the
step is repeated several times at the Llama-3-8B MLP shape (T = 8192,
d = 4096, f = 14336, r = 16; bf16 and 4-bit base weights) and at a small
ragged one, in both workspace strategies, and the fused q/k/v step at the
Llama-3-8B attention shapes, and compared on the device."""
import pytest

import lora_linear_fwd_amd as L
from lora_inputs import gen_linear, gen_mlp

from gpu_helpers import dev, log, mlp_weights

pytestmark = pytest.mark.gpu


def _same(outs, ref, rep):
    import torch
    for k, v in outs.items():
        a, b = v.view(torch.int16), ref[k].view(torch.int16)
        assert torch.equal(a, b), f"rep {rep}: {k} differs in {(a != b).sum().item()} elements"


_SHAPES = {"small": (300, 256, 576, 16, 8, False), "llama3_8b_mlp": (8192, 4096, 14336, 16, 6, False),
           "llama3_8b_mlp_4bit": (8192, 4096, 14336, 16, 4, True)}
# ws "wt": the caller keeps W^T next to each dense weight
_CASES = [(n, ws) for n in _SHAPES for ws in ("fast", "minimal", "wt")
          if not (_SHAPES[n][5] and ws == "wt")]


@pytest.mark.parametrize("name,ws", _CASES, ids=[f"{n}-{w}" for n, w in _CASES])
def test_mlp_step_bitwise_reproducible(name, ws):
    import torch
    T, d, f, r, reps, q4 = _SHAPES[name]
    log(f"determinism: T={T} d={d} f={f} r={r} ws={ws} reps={reps} q4={q4}")
    mi = gen_mlp(T, d, f, r, 16.0, "bf16", seed=51, q4=q4)
    W, _ = mlp_weights(mi)
    if ws == "wt":
        W = {p: L.with_transpose(v) for p, v in W.items()}
    wfmt = L._wfmt(W["gate"])
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
    flag = L.LORA_WS_MINIMAL if ws == "minimal" else 0
    nf = L.workspace_bytes(L.OP_MLP_FWD | flag, L.LORA_BF16, wfmt, T, d, f, r)
    nb = L.workspace_bytes(L.OP_MLP_BWD | flag, L.LORA_BF16, wfmt, T, d, f, r)
    wsb = torch.empty(max(nf, nb), dtype=torch.uint8, device="cuda")
    ref = None
    for rep in range(reps):
        Y, e, g = L.lora_swiglu_mlp_fwd(X, W, A, B, mi.alpha, workspace=wsb[:nf])
        grads = L.lora_swiglu_mlp_bwd(X, W, A, B, mi.alpha, e, g, dY, workspace=wsb[:nb])
        outs = {"Y": Y, "e": e, "g": g, **grads}
        torch.cuda.synchronize()
        if ref is None:
            ref = {k: v.clone() for k, v in outs.items()}
            continue
        _same(outs, ref, rep)


def test_qkv_step_bitwise_reproducible():
    """Fused q/k/v projections (three weight segments in one GEMM) at the
    Llama-3-8B attention shapes (T = 8192, k = 4096, q 4096, k/v 1024, r = 64),
    forward + backward with dX accumulated onto an existing gradient."""
    import torch
    T, k, nq, nkv, r, reps = 8192, 4096, 4096, 1024, 64, 4
    log(f"determinism: qkv T={T} k={k} nq={nq} nkv={nkv} r={r} reps={reps}")
    lis = {p: gen_linear(T, k, n, r, 16.0, "bf16", seed=70 + i)
           for i, (p, n) in enumerate((("q", nq), ("k", nkv), ("v", nkv)))}
    X = dev(lis["q"].X, "bf16")
    W = {p: dev(li.W, "bf16") for p, li in lis.items()}
    A = {p: dev(li.A, "bf16") for p, li in lis.items()}
    B = {p: dev(li.B, "bf16") for p, li in lis.items()}
    dY = {p: dev(li.dY, "bf16") for p, li in lis.items()}
    dX0 = dev(lis["k"].X, "bf16")
    ref = None
    for rep in range(reps):
        o = L.lora_qkv_fwd(X, W, A, B, 16.0)
        dX = dX0.clone()
        gr = L.lora_qkv_bwd(X, W, A, B, 16.0, dY, dX=dX, accumulate_dx=True)
        outs = {**{p: o[p] for p in ("q", "k", "v")}, **{kk: v for kk, v in gr.items() if v is not None}}
        torch.cuda.synchronize()
        if ref is None:
            ref = {kk: v.clone() for kk, v in outs.items()}
            continue
        _same(outs, ref, rep)
