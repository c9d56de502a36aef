"""GPU parity where operands pass 2 GiB, the range of one buffer descriptor.

The GEMMs address every operand through descriptors based at the current
tile (token rows) or the current K step (the backward's weight rows), so
no offset grows with the tensor size.  These cases would read zeros past
2^31 bytes with tensor-wide offsets:
  - the MLP backward's [de | dg] operand ([T x 2f] bf16) past 2 GiB, with a
    small hidden size so the oracle stays cheap: T = 262,437 tokens (a
    ragged last tile), d = 64, f = 4096;
  - one linear layer whose weight [n x k] bf16 passes 2 GiB (n = 139,264,
    k = 8192), read as stored by the backward dX GEMM (K = n rows).
Row-local outputs are checked against the float64 oracle on whole tile
bands and random rows (the linear layer on every row), the adapter
gradients in full (summed over token chunks: they are sums over tokens)."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import _normal, _rngs, _uniform, gen_mlp

from gpu_helpers import check, dev, host, log

pytestmark = [pytest.mark.gpu, pytest.mark.slow]


def band_rows(T, seed, band=256, n=40):
    r = np.random.default_rng(seed)
    nb = (T + band - 1) // band
    bands = [np.arange(b * band, min(T, (b + 1) * band))
             for b in sorted({0, int(r.integers(1, nb - 1)), nb - 1})]
    return np.unique(np.concatenate(bands + [r.integers(0, T, n)]))


def test_mlp_backward_operand_past_2gib():
    import torch
    T, d, f, r, alpha = 262437, 64, 4096, 16, 16.0
    assert T * 2 * f * 2 > 2 ** 31
    log(f"mlp T={T} d={d} f={f} r={r}: generating inputs")
    mi = gen_mlp(T, d, f, r, alpha, "bf16", seed=91)
    s = oracle.scaling(alpha, r)
    W = {p: dev(mi.W[p], "bf16") for p in mi.W}
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    X, dY = dev(mi.X, "bf16"), dev(mi.dY, "bf16")
    log("mlp: GPU forward + backward")
    Y, e, g = L.lora_swiglu_mlp_fwd(X, W, A, B, alpha)
    grads = L.lora_swiglu_mlp_bwd(X, W, A, B, alpha, e, g, dY)
    torch.cuda.synchronize()
    rows = band_rows(T, seed=92)
    rt = torch.from_numpy(rows).to("cuda")
    log(f"mlp: oracle on {len(rows)} rows")
    Yr, er, gr = oracle.mlp_fwd(mi.X[rows], mi.W, mi.A, mi.B, s)
    check("Y[rows]", host(Y[rt]), Yr, "bf16")
    check("e[rows]", host(e[rt]), er, "bf16")
    check("g[rows]", host(g[rt]), gr, "bf16")
    dXr = oracle.mlp_bwd(mi.X[rows], mi.W, mi.A, mi.B, s, mi.dY[rows])["dX"]
    check("dX[rows]", host(grads["dX"][rt]), dXr, "bf16")
    del Y, e, g
    log("mlp: oracle adapter gradients, summed over token chunks")
    ref = None
    for c0 in range(0, T, 16384):
        part = oracle.mlp_bwd(mi.X[c0:c0 + 16384], mi.W, mi.A, mi.B, s, mi.dY[c0:c0 + 16384],
                              want_dx=False)
        part = {k: v for k, v in part.items() if v is not None}
        ref = part if ref is None else {k: ref[k] + part[k] for k in ref}
    for k, v in ref.items():
        check(k, host(grads[k]), v, "bf16")


def _weight_chunk(c, rows, k):
    # seeded per chunk so the oracle regenerates exactly the uploaded values
    return _normal(np.random.Generator(np.random.PCG64(7000 + c)), (rows, k), 0.02, "bf16")


def test_linear_weight_past_2gib():
    import torch
    T, k, n, r, alpha = 300, 8192, 139264, 8, 16.0
    CH = 8192
    assert n * k * 2 > 2 ** 31
    log(f"linear T={T} k={k} n={n} r={r}: uploading the weight in {n // CH} chunks")
    W = torch.empty((n, k), dtype=torch.bfloat16, device="cuda")
    for c in range(n // CH):
        W[c * CH:(c + 1) * CH] = torch.from_numpy(_weight_chunk(c, CH, k)).to(torch.bfloat16)
    rx, ra, rb, rdy = _rngs(93, 4)
    Xh = _normal(rx, (T, k), 1.0, "bf16")
    Ah = _uniform(ra, (r, k), 1.0 / np.sqrt(k), "bf16")
    Bh = _normal(rb, (n, r), 0.02, "bf16")
    dYh = _normal(rdy, (T, n), 1.0, "bf16")
    X, A, B, dY = (dev(v, "bf16") for v in (Xh, Ah, Bh, dYh))
    log("linear: GPU forward + backward")
    Y = L.lora_linear_fwd(X, W, A, B, alpha)
    dX, dA, dB = L.lora_linear_bwd(X, W, A, B, alpha, dY)
    torch.cuda.synchronize()
    del W
    s = oracle.scaling(alpha, r)
    log("linear: oracle over weight chunks (regenerated): every output is a sum of")
    log("        per-chunk oracle calls (Y by columns, dX and dA summed, dB by rows)")
    Yr = np.empty((T, n))
    dXr = np.zeros((T, k))
    dAr = np.zeros((r, k))
    dBr = np.empty((n, r))
    for c in range(n // CH):
        sl = slice(c * CH, (c + 1) * CH)
        Wc = _weight_chunk(c, CH, k)
        Yr[:, sl] = oracle.linear_fwd(Xh, Wc, Ah, Bh[sl], s)
        dXc, dAc, dBc = oracle.linear_bwd(Xh, Wc, Ah, Bh[sl], s, dYh[:, sl])
        dXr += dXc
        dAr += dAc
        dBr[sl] = dBc
    check("Y", host(Y), Yr, "bf16")
    check("dX", host(dX), dXr, "bf16")
    check("dA", host(dA), dAr, "bf16")
    check("dB", host(dB), dBr, "bf16")
