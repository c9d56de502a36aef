"""Bitwise reproducibility of the LoRA-SwiGLU MLP step at full size.

Every reduction in the library runs in a fixed order, so repeated forward +
backward calls on the same inputs must give identical bits.  A race in a
GEMM pipeline (a stage refilled while another wave still reads it) shows up
here as rare differences that a tolerance-based parity check can miss, so the
step is repeated several times at the Llama-3-8B MLP shape (T = 8192,
d = 4096, f = 14336, r = 16) and at a small ragged one, in both workspace
strategies, and compared on the device."""
import pytest

import lora_linear_fwd_amd as L
from lora_inputs import gen_mlp

from gpu_helpers import dev, log, mlp_weights

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("ws", ["fast", "minimal"])
@pytest.mark.parametrize("shape", [(300, 256, 576, 16, 8), (8192, 4096, 14336, 16, 6)],
                         ids=["small", "llama3_8b_mlp"])
def test_mlp_step_bitwise_reproducible(shape, ws):
    import torch
    T, d, f, r, reps = shape
    log(f"determinism: T={T} d={d} f={f} r={r} ws={ws} reps={reps}")
    mi = gen_mlp(T, d, f, r, 16.0, "bf16", seed=51)
    W, _ = mlp_weights(mi)
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
    flag = L.LORA_WS_MINIMAL if ws == "minimal" else 0
    nf = L.workspace_bytes(L.OP_MLP_FWD | flag, L.LORA_BF16, 0, T, d, f, r)
    nb = L.workspace_bytes(L.OP_MLP_BWD | flag, L.LORA_BF16, 0, T, d, f, r)
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
        for k, v in outs.items():
            assert torch.equal(v.view(torch.int16), ref[k].view(torch.int16)), \
                f"rep {rep}: {k} differs in {(v.view(torch.int16) != ref[k].view(torch.int16)).sum().item()} elements"
