"""GPU parity of lora_merge (W' = W + sign s B A) against the float64 oracle,
and the merged-forward invariant on the GPU: the LoRA layer's output equals
a plain linear layer with the merged weight."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import gen_linear, to_bf16_values

from gpu_helpers import check, dev, host, linear_weight, log

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


@pytest.mark.parametrize("shape", [(100, 72, 16), (256, 320, 3), (64, 64, 128), (130, 200, 8)],
                         ids=lambda s: "x".join(map(str, s)))
def test_merge_bf16_within_one_rounding(shape):
    n, k, r = shape
    log(f"merge bf16 n={n} k={k} r={r}")
    li = gen_linear(1, k, n, r, 16.0, "bf16", seed=n + k + r, b_std=0.5)
    s = oracle.scaling(li.alpha, li.r)
    W, A, B = (dev(v, "bf16") for v in (li.W, li.A, li.B))
    out = L.lora_merge(W, A, B, li.alpha)
    _sync()
    ref = oracle.merged_weight(li.W, li.A, li.B, s)
    got = host(out).astype(np.float64)
    # one bf16 rounding (at most one unit of the exact result's last place)
    # of an fp32 sum whose error is bounded by r + 1 fp32 roundings of the
    # magnitudes involved (the bound matters only where W and s B A cancel)
    ulp = np.exp2(np.floor(np.log2(np.maximum(np.abs(ref), 1e-30))) - 7)
    mag = np.abs(li.W.astype(np.float64)) + s * (np.abs(li.B.astype(np.float64))
                                                 @ np.abs(li.A.astype(np.float64)))
    bound = ulp + (r + 1) * 2.0 ** -24 * mag
    assert np.all(np.abs(got - ref) <= bound), np.max(np.abs(got - ref) / bound)
    check("W'", got, ref, "bf16")


def test_merge_fp32():
    li = gen_linear(1, 100, 70, 5, 16.0, "f32", seed=3, b_std=0.5)
    s = oracle.scaling(li.alpha, li.r)
    W, A, B = (dev(v, "f32") for v in (li.W, li.A, li.B))
    out = L.lora_merge(W, A, B, li.alpha)
    _sync()
    check("W' fp32", host(out), oracle.merged_weight(li.W, li.A, li.B, s), "f32")


def test_merge_q4():
    li = gen_linear(1, 256, 136, 16, 16.0, "bf16", seed=5, q4=True, b_std=0.5)
    s = oracle.scaling(li.alpha, li.r)
    Wd, Wref = linear_weight(li)
    A, B = dev(li.A, "bf16"), dev(li.B, "bf16")
    out = L.lora_merge(Wd, A, B, li.alpha)
    _sync()
    check("W' (4-bit base)", host(out), oracle.merged_weight(Wref, li.A, li.B, s), "bf16")


def test_unmerge_inverts_merge():
    li = gen_linear(1, 128, 96, 8, 16.0, "bf16", seed=7, b_std=0.5)
    W, A, B = (dev(v, "bf16") for v in (li.W, li.A, li.B))
    back = L.lora_merge(L.lora_merge(W, A, B, li.alpha), A, B, li.alpha, sign=-1)
    _sync()
    check("unmerge(merge(W))", host(back), li.W, "bf16")


def test_merged_forward_invariant_on_gpu():
    """X W'^T (merged weight, no adapter) = X W^T + s (X A^T) B^T."""
    import torch
    li = gen_linear(300, 320, 264, 16, 16.0, "bf16", seed=9, b_std=1.0)
    s = oracle.scaling(li.alpha, li.r)
    X, W, A, B = (dev(v, "bf16") for v in (li.X, li.W, li.A, li.B))
    Y = L.lora_linear_fwd(X, W, A, B, li.alpha)
    Wm = L.lora_merge(W, A, B, li.alpha)
    Ym = L.lora_linear_fwd(X, Wm, A, torch.zeros_like(B), li.alpha)
    _sync()
    check("merged forward vs LoRA forward", host(Ym), host(Y).astype(np.float64), "bf16")
    check("merged forward vs oracle", host(Ym), oracle.linear_fwd(li.X, li.W, li.A, li.B, s), "bf16")
