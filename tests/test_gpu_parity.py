"""GPU parity: liblora (through its C ABI) against the float64 CPU oracle on
the same seeded inputs, at sizes the oracle finishes in seconds that still
span several 256 x 256 x 64 tiles with ragged tails.  Tolerances: 2e-2
relative Frobenius error per tensor for bf16, 1e-4 for fp32, bit-exact for
the 4-bit decode."""
import numpy as np
import pytest

import lora_linear_fwd_amd as L
import oracle
from lora_inputs import bf16_bits_of, gen_linear, gen_mlp

from gpu_helpers import check, dev, host, linear_weight, log, mlp_weights

pytestmark = pytest.mark.gpu


def _sync():
    import torch
    torch.cuda.synchronize()


# the two workspace strategies: "fast" (weight copied transposed / decoded
# into the workspace, NT GEMMs) and "minimal" (weight read in place: NN
# GEMMs for dX, 4-bit codes decoded inside the GEMM); for dense weights also
# "wt": the caller keeps W^T next to W (the backward runs the NT form on it)
WS_MODES = ["fast", "minimal"]
DENSE_MODES = WS_MODES + ["wt"]


def run_linear(li, need_dx=True, ws="fast"):
    Wd, Wref = linear_weight(li)
    if ws == "wt":
        Wd = L.with_transpose(Wd)
    X, A, B, dY = (dev(v, li.dtype) for v in (li.X, li.A, li.B, li.dY))
    mw = ws == "minimal"
    Y = L.lora_linear_fwd(X, Wd, A, B, li.alpha, minimal_workspace=mw)
    dX, dA, dB = L.lora_linear_bwd(X, Wd, A, B, li.alpha, dY, need_dx=need_dx,
                                   minimal_workspace=mw)
    _sync()
    return Wref, (Y, dX, dA, dB)


def check_linear(li, need_dx=True, ws="fast"):
    s = oracle.scaling(li.alpha, li.r)
    Wref, (Y, dX, dA, dB) = run_linear(li, need_dx, ws)
    Yr = oracle.linear_fwd(li.X, Wref, li.A, li.B, s)
    dXr, dAr, dBr = oracle.linear_bwd(li.X, Wref, li.A, li.B, s, li.dY)
    check("Y", host(Y), Yr, li.dtype)
    if need_dx:
        check("dX", host(dX), dXr, li.dtype)
    check("dA", host(dA), dAr, li.dtype)
    check("dB", host(dB), dBr, li.dtype)


LINEAR_SHAPES = [
    # T, k, n, r : several tiles, ragged M/N/K tails, every side-width path
    (300, 320, 520, 16),
    (37, 72, 40, 3),
    (513, 128, 264, 32),
    (260, 256, 136, 64),
    (130, 64, 72, 128),
    (257, 136, 256, 8),
]


@pytest.mark.parametrize("ws", DENSE_MODES)
@pytest.mark.parametrize("shape", LINEAR_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_linear_bf16(shape, ws):
    T, k, n, r = shape
    log(f"linear bf16 T={T} k={k} n={n} r={r} ws={ws}")
    check_linear(gen_linear(T, k, n, r, 16.0, "bf16", seed=T + k + n + r), ws=ws)


@pytest.mark.parametrize("shape", [(300, 320, 520, 16), (260, 256, 136, 64)],
                         ids=lambda s: "x".join(map(str, s)))
def test_linear_bf16_lora_dominant(shape):
    # B ~ N(0,1): the adapter term is larger than the base term, so a wrong
    # LoRA product cannot hide under the 2e-2 tolerance of Y or dX
    T, k, n, r = shape
    log(f"linear bf16 lora-dominant T={T} k={k} n={n} r={r}")
    check_linear(gen_linear(T, k, n, r, 16.0, "bf16", seed=7, b_std=1.0))


def test_linear_bf16_without_dx():
    log("linear bf16 dX=NULL")
    check_linear(gen_linear(300, 320, 264, 16, 16.0, "bf16", seed=3), need_dx=False)


@pytest.mark.parametrize("shape", [(256, 512, 512, 8), (37, 50, 29, 3), (300, 100, 260, 17)],
                         ids=lambda s: "x".join(map(str, s)))
def test_linear_fp32(shape):
    T, k, n, r = shape
    log(f"linear fp32 T={T} k={k} n={n} r={r}")
    check_linear(gen_linear(T, k, n, r, 16.0, "f32", seed=T * 3 + 1))


@pytest.mark.parametrize("ws", WS_MODES)
def test_linear_q4(ws):
    log(f"linear q4 T=300 k=320 n=264 r=16 ws={ws}")
    check_linear(gen_linear(300, 320, 264, 16, 16.0, "bf16", seed=11, q4=True), ws=ws)
    check_linear(gen_linear(77, 128, 136, 16, 16.0, "bf16", seed=12, q4=True, b_std=1.0), ws=ws)


# one token and the narrowest features the bf16 path takes (multiples of 8):
# every GEMM, rank-r and reduction kernel runs on a single partial tile (the
# last shape: a wide rank, whose rank-r passes take the 128-token blocks)
TINY_LINEAR = [(1, 8, 8, 1), (1, 8, 16, 2), (3, 24, 8, 5), (2, 64, 72, 64)]


@pytest.mark.parametrize("ws", DENSE_MODES)
@pytest.mark.parametrize("shape", TINY_LINEAR, ids=lambda s: "x".join(map(str, s)))
def test_linear_bf16_tiny(shape, ws):
    T, k, n, r = shape
    log(f"linear bf16 tiny T={T} k={k} n={n} r={r} ws={ws}")
    check_linear(gen_linear(T, k, n, r, 16.0, "bf16", seed=T + k + n + r), ws=ws)


def test_linear_B_zero_is_base_layer():
    li = gen_linear(300, 320, 264, 16, 16.0, "bf16", seed=5)
    li.B = np.zeros_like(li.B)
    Wref, (Y, dX, dA, dB) = run_linear(li)
    check("Y(B=0)", host(Y), li.X.astype(np.float64) @ li.W.T.astype(np.float64), "bf16")
    assert np.array_equal(host(dA), np.zeros_like(li.A)), "dA must be exactly 0 when B = 0"
    check("dX(B=0)", host(dX), li.dY.astype(np.float64) @ li.W.astype(np.float64), "bf16")


def test_linear_T_zero():
    import torch
    li = gen_linear(1, 64, 64, 8, 16.0, "bf16")
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    dY = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    W, A, B = (dev(v, "bf16") for v in (li.W, li.A, li.B))
    Y = L.lora_linear_fwd(X, W, A, B, 16.0)
    dA = torch.full_like(A, 7.0)
    dB = torch.full_like(B, 7.0)
    _, dA, dB = L.lora_linear_bwd(X, W, A, B, 16.0, dY, dA=dA, dB=dB)
    _sync()
    assert Y.shape == (0, 64)
    assert torch.count_nonzero(dA).item() == 0 and torch.count_nonzero(dB).item() == 0


def test_linear_accumulate_dx_sums_projections():
    # q/k/v-style: three projections of one X; dX accumulates their inputs' grads
    T, k = 200, 128
    lis = [gen_linear(T, k, n, 16, 16.0, "bf16", seed=40 + i) for i, n in enumerate((128, 64, 64))]
    X = dev(lis[0].X, "bf16")
    import torch
    dX = torch.zeros((T, k), dtype=torch.bfloat16, device="cuda")
    ref = np.zeros((T, k))
    for i, li in enumerate(lis):
        W, A, B, dY = (dev(v, "bf16") for v in (li.W, li.A, li.B, li.dY))
        L.lora_linear_bwd(X, W, A, B, 16.0, dY, dX=dX, accumulate_dx=i > 0)
        ref += oracle.linear_bwd(lis[0].X, li.W, li.A, li.B, 1.0, li.dY)[0]
    _sync()
    check("dX(q+k+v)", host(dX), ref, "bf16")


def test_linear_deterministic():
    li = gen_linear(300, 320, 520, 16, 16.0, "bf16", seed=9)
    _, o1 = run_linear(li)
    _, o2 = run_linear(li)
    for a, b in zip(o1, o2):
        assert np.array_equal(host(a), host(b))


# ------------------------------------------------------------------ MLP
def run_mlp(mi, need_dx=True, ws="fast"):
    Wd, Wref = mlp_weights(mi)
    if ws == "wt":
        Wd = {p: L.with_transpose(v) for p, v in Wd.items()}
    X, dY = dev(mi.X, mi.dtype), dev(mi.dY, mi.dtype)
    A = {p: dev(mi.A[p], mi.dtype) for p in mi.A}
    B = {p: dev(mi.B[p], mi.dtype) for p in mi.B}
    mw = ws == "minimal"
    Y, e, g = L.lora_swiglu_mlp_fwd(X, Wd, A, B, mi.alpha, minimal_workspace=mw)
    grads = L.lora_swiglu_mlp_bwd(X, Wd, A, B, mi.alpha, e, g, dY, need_dx=need_dx,
                                  minimal_workspace=mw)
    _sync()
    return Wref, Y, e, g, grads


def check_mlp(mi, need_dx=True, ws="fast"):
    s = oracle.scaling(mi.alpha, mi.r)
    Wref, Y, e, g, grads = run_mlp(mi, need_dx, ws)
    Yr, er, gr = oracle.mlp_fwd(mi.X, Wref, mi.A, mi.B, s)
    check("Y", host(Y), Yr, mi.dtype)
    check("e", host(e), er, mi.dtype)
    check("g", host(g), gr, mi.dtype)
    ref = oracle.mlp_bwd(mi.X, Wref, mi.A, mi.B, s, mi.dY, want_dx=need_dx)
    for key, val in ref.items():
        if val is None:
            continue
        check(key, host(grads[key]), val, mi.dtype)


MLP_SHAPES = [
    # T, d, f, r  (with "wt", f % 64 == 0 runs the gate/up backward as one NT
    # product over [Wg^T | Wu^T]; other f read the gate/up weights as stored)
    (300, 256, 520, 16),
    (300, 264, 512, 16),
    (37, 64, 72, 3),
    (260, 128, 264, 64),
    (513, 136, 256, 8),
    (200, 192, 392, 24),    # 16 < r <= 32: the dual rank-r passes, not the fused epilogue
    (130, 256, 512, 32),
    (70, 64, 136, 128),     # widest side operands (2 r = 256)
    (130, 128, 200, 40),    # wide rank not a multiple of 16: one 2r-wide pass over [de | dg]
]


@pytest.mark.parametrize("ws", DENSE_MODES)
@pytest.mark.parametrize("shape", MLP_SHAPES, ids=lambda s: "x".join(map(str, s)))
def test_mlp_bf16(shape, ws):
    T, d, f, r = shape
    log(f"mlp bf16 T={T} d={d} f={f} r={r} ws={ws}")
    check_mlp(gen_mlp(T, d, f, r, 16.0, "bf16", seed=T + d + f + r), ws=ws)


@pytest.mark.parametrize("ws", ["fast", "wt"])
def test_mlp_bf16_lora_dominant(ws):
    log(f"mlp bf16 lora-dominant ws={ws}")
    check_mlp(gen_mlp(300, 256, 512, 16, 16.0, "bf16", seed=21, b_std=1.0), ws=ws)


def test_mlp_bf16_without_dx():
    check_mlp(gen_mlp(300, 256, 520, 16, 16.0, "bf16", seed=22), need_dx=False)


def test_mlp_fp32():
    log("mlp fp32")
    check_mlp(gen_mlp(67, 48, 80, 5, 16.0, "f32", seed=23))


@pytest.mark.parametrize("ws", WS_MODES)
def test_mlp_q4(ws):
    log(f"mlp q4 T=300 d=256 f=576 r=16 ws={ws}")
    check_mlp(gen_mlp(300, 256, 576, 16, 16.0, "bf16", seed=24, q4=True), ws=ws)
    check_mlp(gen_mlp(70, 128, 192, 16, 16.0, "bf16", seed=25, q4=True, b_std=1.0), ws=ws)


# the same for the MLP; the last two: wide ranks (saved h, 128-token rank-r
# blocks; a multiple of 16 with the block-by-block passes, and one that is not)
TINY_MLP = [(1, 8, 8, 1), (2, 16, 24, 2), (5, 8, 136, 16), (3, 16, 64, 64), (2, 8, 72, 40)]


@pytest.mark.parametrize("ws", DENSE_MODES)
@pytest.mark.parametrize("shape", TINY_MLP, ids=lambda s: "x".join(map(str, s)))
def test_mlp_bf16_tiny(shape, ws):
    T, d, f, r = shape
    log(f"mlp bf16 tiny T={T} d={d} f={f} r={r} ws={ws}")
    check_mlp(gen_mlp(T, d, f, r, 16.0, "bf16", seed=T + d + f + r), ws=ws)


def test_mlp_T_zero():
    import torch
    mi = gen_mlp(1, 64, 128, 8, 16.0, "bf16")
    Wd, _ = mlp_weights(mi)
    A = {p: dev(mi.A[p], "bf16") for p in mi.A}
    B = {p: dev(mi.B[p], "bf16") for p in mi.B}
    X = torch.empty((0, 64), dtype=torch.bfloat16, device="cuda")
    Y, e, g = L.lora_swiglu_mlp_fwd(X, Wd, A, B, 16.0)
    out = {k: torch.full_like(v, 3.0) for k, v in
           [("dA_" + p, A[p]) for p in A] + [("dB_" + p, B[p]) for p in B]}
    grads = L.lora_swiglu_mlp_bwd(X, Wd, A, B, 16.0, e, g, X, out=out)
    _sync()
    for k_, v in grads.items():
        if k_ != "dX":
            assert torch.count_nonzero(v).item() == 0, k_


# ------------------------------------------------------------- 4-bit decode
@pytest.mark.parametrize("nk", [(264, 320), (1, 64), (4096, 1024)], ids=str)
def test_dequant4_bit_exact(nk):
    n, k = nk
    li = gen_linear(1, k, n, 1, 1.0, "bf16", seed=n + k, q4=True)
    q = li.q4
    out = L.lora_dequant4(L.to_device_q4(q))
    _sync()
    import torch
    got = out.view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.decode_q4_bits(q.codes, q.absmax, q.codebook, n, k)
    assert np.array_equal(got, ref)


def test_dequant4_hand_fixture_on_gpu():
    # the double-rounding case pinned in the oracle tests, decoded on the GPU
    import torch
    cb = np.zeros(16, np.float32)
    cb[7], cb[8], cb[15] = 1 + 2 ** -8, 1 + 3 * 2 ** -8, float.fromhex("0x1.00fffep+0")
    codes = np.zeros((1, 64), np.uint8)
    codes[0, :3] = [7, 8, 15]
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    am = np.array([float.fromhex("0x1.000002p+0")], np.float32)
    from lora_inputs import Q4Weight
    q = L.to_device_q4(Q4Weight(1, 64, packed, am, cb))
    got = L.lora_dequant4(q).view(torch.int16).cpu().numpy().view(np.uint16)
    ref = oracle.decode_q4_bits(packed, am, cb, 1, 64)
    assert np.array_equal(got, ref)
    assert got[0, 2] == 0x3F80
