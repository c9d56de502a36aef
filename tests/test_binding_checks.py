"""The Python binding checks every tensor against the sizes it derives
(shape, dtype, device, contiguity) before it calls the library: the C ABI
takes bare pointers, so a wrong-shaped or strided tensor would otherwise be
read or written out of bounds.  These run on the CPU: every call here must
raise ValueError before any library call (CPU tensors are refused last, as
not being on a GPU)."""
import pytest
import torch

import lora_linear_fwd_amd as L

bf = torch.bfloat16


def lin(T=8, k=64, n=32, r=4, dt=bf):
    return (torch.zeros(T, k, dtype=dt), torch.zeros(n, k, dtype=dt), torch.zeros(r, k, dtype=dt),
            torch.zeros(n, r, dtype=dt))


def test_linear_fwd_checks():
    X, W, A, B = lin()
    with pytest.raises(ValueError, match="on a GPU"):       # everything else is right
        L.lora_linear_fwd(X, W, A, B, 16.0)
    with pytest.raises(ValueError, match="A has shape"):
        L.lora_linear_fwd(X, W, torch.zeros(4, 63, dtype=bf), B, 16.0)
    with pytest.raises(ValueError, match="B has shape"):
        L.lora_linear_fwd(X, W, A, torch.zeros(32, 5, dtype=bf), 16.0)
    with pytest.raises(ValueError, match="W has shape"):
        L.lora_linear_fwd(X, torch.zeros(32, 48, dtype=bf), A, B, 16.0)
    with pytest.raises(ValueError, match="dtype"):
        L.lora_linear_fwd(X, W.float(), A, B, 16.0)
    with pytest.raises(ValueError, match="Y has shape"):
        L.lora_linear_fwd(X, W, A, B, 16.0, Y=torch.zeros(8, 33, dtype=bf))
    with pytest.raises(ValueError, match="contiguous"):      # a transposed view
        L.lora_linear_fwd(X, torch.zeros(64, 32, dtype=bf).t(), A, B, 16.0)
    with pytest.raises(ValueError, match="contiguous"):
        L.lora_linear_fwd(torch.zeros(64, 8, dtype=bf).t(), W, A, B, 16.0)


def test_linear_bwd_checks():
    X, W, A, B = lin()
    dY = torch.zeros(8, 32, dtype=bf)
    with pytest.raises(ValueError, match="on a GPU"):
        L.lora_linear_bwd(X, W, A, B, 16.0, dY)
    with pytest.raises(ValueError, match="dY has shape"):
        L.lora_linear_bwd(X, W, A, B, 16.0, torch.zeros(8, 64, dtype=bf))
    with pytest.raises(ValueError, match="dX has shape"):
        L.lora_linear_bwd(X, W, A, B, 16.0, dY, dX=torch.zeros(8, 32, dtype=bf))
    with pytest.raises(ValueError, match="accumulate_dx needs dX"):
        L.lora_linear_bwd(X, W, A, B, 16.0, dY, accumulate_dx=True)
    with pytest.raises(ValueError, match="dA has shape"):
        L.lora_linear_bwd(X, W, A, B, 16.0, dY, dA=torch.zeros(4, 32, dtype=bf))


def mlp(T=8, d=64, f=128, r=4):
    W = {"gate": torch.zeros(f, d, dtype=bf), "up": torch.zeros(f, d, dtype=bf),
         "down": torch.zeros(d, f, dtype=bf)}
    A = {"gate": torch.zeros(r, d, dtype=bf), "up": torch.zeros(r, d, dtype=bf),
         "down": torch.zeros(r, f, dtype=bf)}
    B = {"gate": torch.zeros(f, r, dtype=bf), "up": torch.zeros(f, r, dtype=bf),
         "down": torch.zeros(d, r, dtype=bf)}
    return torch.zeros(T, d, dtype=bf), W, A, B


def test_mlp_checks():
    X, W, A, B = mlp()
    with pytest.raises(ValueError, match="on a GPU"):
        L.lora_swiglu_mlp_fwd(X, W, A, B, 16.0)
    bad = dict(W, down=torch.zeros(64, 64, dtype=bf))            # down must be [d, f]
    with pytest.raises(ValueError, match="W_down has shape"):
        L.lora_swiglu_mlp_fwd(X, bad, A, B, 16.0)
    badA = dict(A, up=torch.zeros(5, 64, dtype=bf))              # ranks must agree
    with pytest.raises(ValueError, match="A_up has shape"):
        L.lora_swiglu_mlp_fwd(X, W, badA, B, 16.0)
    with pytest.raises(ValueError, match="e has shape"):
        L.lora_swiglu_mlp_fwd(X, W, A, B, 16.0, e=torch.zeros(8, 64, dtype=bf))
    e = torch.zeros(8, 128, dtype=bf)
    with pytest.raises(ValueError, match="on a GPU"):
        L.lora_swiglu_mlp_bwd(X, W, A, B, 16.0, e, e, X)
    with pytest.raises(ValueError, match="g has shape"):
        L.lora_swiglu_mlp_bwd(X, W, A, B, 16.0, e, torch.zeros(8, 127, dtype=bf), X)
    with pytest.raises(ValueError, match="dB_down has shape"):
        L.lora_swiglu_mlp_bwd(X, W, A, B, 16.0, e, e, X,
                              out={"dB_down": torch.zeros(128, 4, dtype=bf)})
    with pytest.raises(ValueError, match="keys"):
        L.lora_swiglu_mlp_fwd(X, {"gate": W["gate"]}, A, B, 16.0)


def test_q4_container_checks():
    n, k = 32, 128
    q = L.Q4Weight(n, k, torch.zeros(n, k // 2, dtype=torch.uint8),
                   torch.zeros(n * k // 64, dtype=torch.float32),
                   torch.zeros(16, dtype=torch.float32))
    X = torch.zeros(8, k, dtype=bf)
    A, B = torch.zeros(4, k, dtype=bf), torch.zeros(n, 4, dtype=bf)
    with pytest.raises(ValueError, match="on a GPU"):
        L.lora_linear_fwd(X, q, A, B, 16.0)
    short = L.Q4Weight(n, k, q.codes[:, :32].contiguous(), q.absmax, q.codebook)
    with pytest.raises(ValueError, match="codes has shape"):
        L.lora_linear_fwd(X, short, A, B, 16.0)
    wrong_am = L.Q4Weight(n, k, q.codes, q.absmax[:-1].contiguous(), q.codebook)
    with pytest.raises(ValueError, match="absmax has shape"):
        L.lora_linear_fwd(X, wrong_am, A, B, 16.0)
    with pytest.raises(ValueError, match="bf16"):
        L.lora_linear_fwd(X.float(), q, A.float(), B.float(), 16.0)
    with pytest.raises(ValueError, match="codebook"):
        L.lora_decode_weight(L.Q4Weight(n, k, q.codes, q.absmax, torch.zeros(8)))


def test_qkv_and_norm_checks():
    X = torch.zeros(8, 64, dtype=bf)
    W = {"q": torch.zeros(64, 64, dtype=bf), "k": torch.zeros(32, 64, dtype=bf),
         "v": torch.zeros(32, 64, dtype=bf)}
    A = {p: torch.zeros(4, 64, dtype=bf) for p in "qkv"}
    B = {p: torch.zeros(W[p].shape[0], 4, dtype=bf) for p in "qkv"}
    with pytest.raises(ValueError, match="on a GPU"):
        L.lora_qkv_fwd(X, W, A, B, 16.0)
    with pytest.raises(ValueError, match="W_v has shape"):
        L.lora_qkv_fwd(X, dict(W, v=torch.zeros(48, 64, dtype=bf)), A, B, 16.0)
    dY = {"q": torch.zeros(8, 64, dtype=bf), "k": torch.zeros(8, 32, dtype=bf),
          "v": torch.zeros(8, 64, dtype=bf)}
    with pytest.raises(ValueError, match="dV has shape"):
        L.lora_qkv_bwd(X, W, A, B, 16.0, dY)
    w = torch.ones(64, dtype=bf)
    with pytest.raises(ValueError, match="on a GPU"):
        L.lora_rmsnorm_fwd(X, w, 1e-5)
    with pytest.raises(ValueError, match="w has shape"):
        L.lora_rmsnorm_fwd(X, torch.ones(63, dtype=bf), 1e-5)
    with pytest.raises(ValueError, match="alias"):
        L.lora_rmsnorm_fwd(X, w, 1e-5, Y=X)
    with pytest.raises(ValueError, match="rstd has shape"):
        L.lora_rmsnorm_bwd(X, w, torch.zeros(7), X)


def test_merge_checks():
    W = torch.zeros(32, 64, dtype=bf)
    A, B = torch.zeros(4, 64, dtype=bf), torch.zeros(32, 4, dtype=bf)
    with pytest.raises(ValueError, match="on a GPU"):
        L.lora_merge(W, A, B, 16.0)
    with pytest.raises(ValueError, match="B has shape"):
        L.lora_merge(W, A, torch.zeros(32, 3, dtype=bf), 16.0)
    with pytest.raises(ValueError, match="out has shape"):
        L.lora_merge(W, A, B, 16.0, out=torch.zeros(64, 32, dtype=bf))
