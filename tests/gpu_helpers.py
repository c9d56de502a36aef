"""Helpers shared by the GPU parity tests: upload seeded inputs through
torch (device memory only) and compare liblora's outputs with the oracle."""
import sys

import numpy as np

import lora_linear_fwd_amd as L
import oracle

BF16_TOL = 2e-2     # relative Frobenius error per output/gradient tensor
F32_TOL = 1e-4
# Element-wise bound beside the Frobenius one, so that an error confined to a
# few tiles (a stale block, a wrong ragged tail) cannot hide in a tensor-wide
# norm: |got - ref| <= ELEM_C * u * (|ref| + rms(ref)) per element, u the unit
# roundoff of the storage type (2^-8 for bf16; 2^-16 for fp32, whose results
# sum thousands of products).  The |ref| term covers the final rounding of
# each output, the rms term the rounding of intermediates (e, g, h, de, dg
# and the rank-r products are stored in bf16) propagated through a K-long
# sum, which scales like the output itself.  ELEM_C = 16 leaves room for the
# largest of millions of such errors; a zeroed or stale element of typical
# size exceeds the bound about 8-fold.
ELEM_C = 16.0
ELEM_U = {"bf16": 2.0 ** -8, "f32": 2.0 ** -16}


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


def elem_ratio(got, ref, dtype):
    """max over elements of |got - ref| / (ELEM_C u (|ref| + rms(ref)))."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    if ref.size == 0:
        return 0.0
    rms = float(np.sqrt(np.mean(ref * ref)))
    bound = ELEM_C * ELEM_U[dtype] * (np.abs(ref) + rms)
    diff = np.abs(got - ref)
    with np.errstate(divide="ignore", invalid="ignore"):
        r = np.where(diff == 0.0, 0.0, diff / bound)
    return float(np.max(r))


def check(name, got, ref, dtype, tol_=None):
    err = oracle.rel_fro(got, ref)
    lim = tol(dtype) if tol_ is None else tol_
    worst = elem_ratio(got, ref, dtype)
    log(f"  {name}: rel_fro={err:.3e} (limit {lim:.0e}), element bound used {worst:.3f}")
    assert np.isfinite(got).all(), f"{name} has non-finite values"
    assert err <= lim, f"{name}: rel_fro {err:.3e} > {lim:.0e}"
    if worst > 1.0:
        got_, ref_ = np.asarray(got, np.float64), np.asarray(ref, np.float64)
        rms = float(np.sqrt(np.mean(ref_ * ref_)))
        bad = np.argwhere(np.abs(got_ - ref_) > ELEM_C * ELEM_U[dtype] * (np.abs(ref_) + rms))
        raise AssertionError(f"{name}: {len(bad)} elements outside the element-wise bound "
                             f"(worst {worst:.2f}x), first at {bad[:4].tolist()}")
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
