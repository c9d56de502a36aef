"""Helpers shared by the GPU parity tests: upload seeded inputs through
torch (device memory only) and compare liblora's outputs with the oracle."""
import sys

import numpy as np

import lora_linear_fwd_amd as L
import oracle

BF16_TOL = 2e-2     # relative Frobenius error per output/gradient tensor
F32_TOL = 1e-4


def log(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def dev(x, dtype):
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    t = t.to(torch.bfloat16) if dtype == "bf16" else t
    return t.to("cuda")


def host(t):
    import torch
    return t.detach().to(torch.float32).cpu().numpy().astype(np.float64)


def tol(dtype):
    return BF16_TOL if dtype == "bf16" else F32_TOL


def check(name, got, ref, dtype, tol_=None):
    err = oracle.rel_fro(got, ref)
    lim = tol(dtype) if tol_ is None else tol_
    log(f"  {name}: rel_fro={err:.3e} (limit {lim:.0e})")
    assert np.isfinite(got).all(), f"{name} has non-finite values"
    assert err <= lim, f"{name}: rel_fro {err:.3e} > {lim:.0e}"
    return err


def linear_weight(li):
    """Device weight (dense tensor or Q4) and the oracle's float64 W."""
    if li.q4 is not None:
        q = li.q4
        Wd = L.to_device_q4(q)
        Wref = oracle.decode_q4_weight(q)
        return Wd, Wref
    return dev(li.W, li.dtype), li.W


def mlp_weights(mi):
    Wd, Wref = {}, {}
    for p in ("gate", "up", "down"):
        if mi.q4:
            q = mi.q4[p]
            Wd[p] = L.to_device_q4(q)
            Wref[p] = oracle.decode_q4_weight(q)
        else:
            Wd[p] = dev(mi.W[p], mi.dtype)
            Wref[p] = mi.W[p]
    return Wd, Wref
