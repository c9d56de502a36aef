"""Pins of the CPU oracle to facts that do not come from the oracle itself.

Each test names what fixes the expected value: the pages' printed worked
example, an invariant the pages state, a closed form, brute force on tiny
inputs, central finite differences, or an independent library routine.
"""
import json
import math
import os

import numpy as np
import pytest

import oracle
from lora_inputs import (bf16_bits_of, gen_linear, gen_mlp, make_absmax_codebook, make_codebook,
                         to_bf16_values)

GOLDEN = os.path.join(os.path.dirname(__file__), "golden")
rng = np.random.default_rng(12345)


def _lin(T=5, k=7, n=6, r=3, seed=1, b_std=0.5):
    g = np.random.default_rng(seed)
    X = g.standard_normal((T, k))
    W = g.standard_normal((n, k)) * 0.3
    A = g.uniform(-1, 1, (r, k))
    B = g.standard_normal((n, r)) * b_std
    dY = g.standard_normal((T, n))
    return X, W, A, B, dY


def _mlp(T=3, d=4, f=6, r=2, seed=2):
    g = np.random.default_rng(seed)
    X = g.standard_normal((T, d))
    shp = {"gate": (f, d), "up": (f, d), "down": (d, f)}
    W = {k: g.standard_normal(v) * 0.4 for k, v in shp.items()}
    A = {k: g.uniform(-1, 1, (r, v[1])) for k, v in shp.items()}
    B = {k: g.standard_normal((v[0], r)) * 0.5 for k, v in shp.items()}
    dY = g.standard_normal((T, d))
    return X, W, A, B, dY


# ----------------------------------------------------------------- printed
def test_trainable_params_printed_example():
    fx = json.load(open(os.path.join(GOLDEN, "trainable_params.json")))
    n, k, r = fx["n"], fx["k"], fx["r"]
    assert n * k == fx["full_params"]
    assert oracle.trainable_params(n, k, r) == fx["lora_params"]
    assert (n * k) // oracle.trainable_params(n, k, r) == fx["reduction"]
    # and it is the element count of the adapter tensors the layer holds
    A = np.zeros((r, k)); B = np.zeros((n, r))
    assert A.size + B.size == fx["lora_params"]


def test_scaling_is_alpha_over_rank():
    assert oracle.scaling(16.0, 8) == 2.0
    assert oracle.scaling(16.0, 16) == 1.0
    assert oracle.scaling(16.0, 64) == 0.25


# -------------------------------------------------------------- invariants
def test_B_zero_gives_base_layer_exactly():
    X, W, A, B, dY = _lin()
    B0 = np.zeros_like(B)
    s = 2.0
    Y = oracle.linear_fwd(X, W, A, B0, s)
    assert np.array_equal(Y, X @ W.T)
    dX, dA, dB = oracle.linear_bwd(X, W, A, B0, s, dY)
    assert np.array_equal(dA, np.zeros_like(A))
    assert np.array_equal(dX, dY @ W)
    assert np.abs(dB).max() > 0     # dB is nonzero even at B = 0


def test_merged_weight_equals_unmerged():
    for (T, k, n, r) in [(5, 7, 6, 3), (9, 16, 24, 4), (4, 8, 8, 8)]:
        X, W, A, B, _ = _lin(T, k, n, r, seed=T + k)
        s = 0.75
        Y = oracle.linear_fwd(X, W, A, B, s)
        Wm = W + s * np.einsum("nq,qk->nk", B, A)
        Ym = X @ Wm.T
        assert oracle.rel_fro(Y, Ym) < 1e-13
        assert oracle.rel_fro(oracle.merged_weight(W, A, B, s), Wm) < 1e-15


def test_forward_brute_force_loops():
    X, W, A, B, _ = _lin(T=3, k=4, n=5, r=2, seed=7)
    s = 1.5
    Y = oracle.linear_fwd(X, W, A, B, s)
    for t in range(3):
        for j in range(5):
            base = sum(X[t, i] * W[j, i] for i in range(4))
            lora = 0.0
            for q in range(2):
                lora += B[j, q] * sum(A[q, i] * X[t, i] for i in range(4))
            assert abs(Y[t, j] - (base + s * lora)) < 1e-12


def test_identity_adapter_reduces_to_plain_gemm():
    # r = k and A = I: X A^T B^T = X B^T, so Y = X (W + s B)^T, a plain GEMM
    g = np.random.default_rng(3)
    T, k, n = 6, 5, 4
    X = g.standard_normal((T, k)); W = g.standard_normal((n, k))
    B = g.standard_normal((n, k))
    Y = oracle.linear_fwd(X, W, np.eye(k), B, 0.5)
    ref = np.array([[sum(X[t, i] * (W[j, i] + 0.5 * B[j, i]) for i in range(k))
                     for j in range(n)] for t in range(T)])
    assert np.abs(Y - ref).max() < 1e-12


def test_linearity_in_x_and_in_s():
    X, W, A, B, _ = _lin()
    Y = oracle.linear_fwd(X, W, A, B, 1.0)
    assert np.array_equal(oracle.linear_fwd(2 * X, W, A, B, 1.0), 2 * Y)
    Y0 = oracle.linear_fwd(X, W, A, B, 0.0)
    Y1 = oracle.linear_fwd(X, W, A, B, 1.0)
    Y3 = oracle.linear_fwd(X, W, A, B, 3.0)
    assert np.abs((Y3 - Y0) - 3 * (Y1 - Y0)).max() < 1e-12


# ------------------------------------------------------ finite differences
def _fd(fun, arr, h=1e-6):
    grad = np.zeros_like(arr)
    it = np.nditer(arr, flags=["multi_index"])
    for _ in it:
        idx = it.multi_index
        old = arr[idx]
        arr[idx] = old + h; fp = fun()
        arr[idx] = old - h; fm = fun()
        arr[idx] = old
        grad[idx] = (fp - fm) / (2 * h)
    return grad


def test_linear_gradients_finite_differences():
    X, W, A, B, dY = _lin(T=4, k=6, n=5, r=2, seed=11)
    s = 2.0
    loss = lambda: float(np.sum(dY * oracle.linear_fwd(X, W, A, B, s)))
    dX, dA, dB = oracle.linear_bwd(X, W, A, B, s, dY)
    for name, arr, got in (("X", X, dX), ("A", A, dA), ("B", B, dB)):
        fd = _fd(loss, arr)
        assert oracle.rel_fro(got, fd) < 1e-7, name


def test_mlp_gradients_finite_differences():
    X, W, A, B, dY = _mlp(T=3, d=4, f=6, r=2, seed=5)
    s = 0.5
    loss = lambda: float(np.sum(dY * oracle.mlp_fwd(X, W, A, B, s)[0]))
    got = oracle.mlp_bwd(X, W, A, B, s, dY)
    assert oracle.rel_fro(got["dX"], _fd(loss, X)) < 1e-7
    for p in ("gate", "up", "down"):
        assert oracle.rel_fro(got["dA_" + p], _fd(loss, A[p])) < 1e-7, p
        assert oracle.rel_fro(got["dB_" + p], _fd(loss, B[p])) < 1e-7, p


def test_mlp_against_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    X, W, A, B, dY = _mlp(T=17, d=24, f=40, r=3, seed=9)
    s = 0.25
    tX = torch.tensor(X, requires_grad=True)
    tA = {k: torch.tensor(v, requires_grad=True) for k, v in A.items()}
    tB = {k: torch.tensor(v, requires_grad=True) for k, v in B.items()}
    tW = {k: torch.tensor(v) for k, v in W.items()}

    def lin(x, p):
        return torch.nn.functional.linear(x, tW[p]) + s * torch.nn.functional.linear(
            torch.nn.functional.linear(x, tA[p]), tB[p])
    e, g = lin(tX, "gate"), lin(tX, "up")
    Y = lin(torch.nn.functional.silu(e) * g, "down")
    Y.backward(torch.tensor(dY))
    ref_Y, ref_e, ref_g = oracle.mlp_fwd(X, W, A, B, s)
    assert oracle.rel_fro(ref_Y, Y.detach().numpy()) < 1e-13
    assert oracle.rel_fro(ref_e, e.detach().numpy()) < 1e-13
    got = oracle.mlp_bwd(X, W, A, B, s, dY)
    assert oracle.rel_fro(got["dX"], tX.grad.numpy()) < 1e-12
    for p in ("gate", "up", "down"):
        assert oracle.rel_fro(got["dA_" + p], tA[p].grad.numpy()) < 1e-12
        assert oracle.rel_fro(got["dB_" + p], tB[p].grad.numpy()) < 1e-12


def test_linear_against_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    X, W, A, B, dY = _lin(T=33, k=20, n=12, r=5, seed=4)
    s = 2.0
    tX, tA, tB = (torch.tensor(v, requires_grad=True) for v in (X, A, B))
    Y = tX @ torch.tensor(W).T + s * (tX @ tA.T) @ tB.T
    Y.backward(torch.tensor(dY))
    dX, dA, dB = oracle.linear_bwd(X, W, A, B, s, dY)
    assert oracle.rel_fro(dX, tX.grad.numpy()) < 1e-13
    assert oracle.rel_fro(dA, tA.grad.numpy()) < 1e-13
    assert oracle.rel_fro(dB, tB.grad.numpy()) < 1e-13


# ------------------------------------------------------------- silu / swiglu
def test_silu_closed_forms():
    from scipy.special import expit
    z = np.linspace(-30, 30, 2001)
    assert np.abs(oracle.sigmoid(z) - expit(z)).max() < 1e-15
    assert oracle.swiglu(np.array([0.0]), np.array([3.0]))[0] == 0.0
    assert oracle.sigmoid(np.array([0.0]))[0] == 0.5
    # silu'(0) = 1/2: with g = 1 and dh = 1, de = silu'(e)
    de, dg = oracle.swiglu_bwd(np.array([0.0]), np.array([1.0]), np.array([1.0]))
    assert de[0] == 0.5 and dg[0] == 0.0
    big = np.array([50.0])
    assert abs(oracle.swiglu(big, np.array([1.0]))[0] - 50.0) < 1e-12
    assert abs(oracle.swiglu(-big, np.array([1.0]))[0]) < 1e-18
    # huge negative gate: no inf * 0
    de, dg = oracle.swiglu_bwd(np.array([-1e4]), np.array([2.0]), np.array([1.0]))
    assert de[0] == 0.0 and np.isfinite(dg[0])


def test_swiglu_derivative_finite_differences():
    e = np.linspace(-6, 6, 61); g = np.cos(e) + 1.5; h = 1e-6
    de, dg = oracle.swiglu_bwd(e, g, np.ones_like(e))
    fd_e = (oracle.swiglu(e + h, g) - oracle.swiglu(e - h, g)) / (2 * h)
    fd_g = (oracle.swiglu(e, g + h) - oracle.swiglu(e, g - h)) / (2 * h)
    assert np.abs(de - fd_e).max() < 1e-8
    assert np.abs(dg - fd_g).max() < 1e-8


# -------------------------------------------------------------- bf16 / 4-bit
def test_bf16_rne_matches_torch():
    torch = pytest.importorskip("torch")
    x = (rng.standard_normal(1_000_000) * np.exp(rng.uniform(-20, 20, 1_000_000))).astype(np.float32)
    # exact ties: low 16 bits == 0x8000, with both parities of bit 16
    ties = (rng.integers(0, 2**31, 20000, dtype=np.uint32) & 0xFFFF0000) | 0x8000
    extra = np.array([0.0, -0.0, np.inf, -np.inf, np.finfo(np.float32).max,
                      -np.finfo(np.float32).max, 1e-40, -1e-40], dtype=np.float32)
    x = np.concatenate([x, ties.view(np.float32), extra])
    x = x[~np.isnan(x)]
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(oracle.bf16_rne_bits(x), ref)


def test_bf16_rne_hand_cases():
    f = lambda v: int(oracle.bf16_rne_bits(np.array([v], dtype=np.float32))[0])
    assert f(1.0) == 0x3F80
    assert f(1.0 + 2**-8) == 0x3F80            # tie, 1.0 is even
    assert f(1.0 + 3 * 2**-8) == 0x3F82        # tie between 0x3F81 and 0x3F82
    assert f(1.0 + 2**-8 + 2**-20) == 0x3F81   # above the tie
    assert f(-2.0) == 0xC000


def test_q4_decode_hand_fixture():
    # codebook entries chosen so that every product below is worked out by hand
    cb = np.array([-1.0, -0.5, -0.25, 0.0, 0.25, 0.5, 1.0, 1 + 2**-8, 1 + 3 * 2**-8,
                   0.75, -0.75, 0.125, -0.125, 0.375, -0.375,
                   float.fromhex("0x1.00fffep+0")], dtype=np.float32)
    n, k = 2, 128
    codes = np.full((n, k), 3, dtype=np.uint8)       # level 0.0 everywhere
    absmax = np.array([2.0, 1.0, 0.5, float.fromhex("0x1.000002p+0")], dtype=np.float32)
    codes[0, 0:4] = [6, 0, 3, 4]       # 1*2, -1*2, 0*2, 0.25*2
    codes[0, 64:70] = [7, 8, 9, 10, 11, 1]
    codes[1, 0:2] = [12, 13]           # row 1 block 0 uses absmax 0.5
    codes[1, 64] = 15                  # double-rounding case
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    # nibble order: element 2j is the low nibble of byte j
    assert packed[0, 0] == 0x06 and packed[0, 1] == 0x43 and packed[0, 32] == 0x87
    bits = oracle.decode_q4_bits(packed, absmax, cb, n, k)
    assert bits.dtype == np.uint16
    assert list(bits[0, 0:4]) == [0x4000, 0xC000, 0x0000, 0x3F00]
    # 1+2^-8 (tie -> even 0x3F80); 1+3*2^-8 (tie -> even 0x3F82); 0.75; -0.75; 0.125; -0.5
    assert list(bits[0, 64:70]) == [0x3F80, 0x3F82, 0x3F40, 0xBF40, 0x3E00, 0xBF00]
    assert list(bits[1, 0:2]) == [0xBD80, 0x3E40]    # -0.0625, 0.1875
    # (1+2^-8-2^-23)*(1+2^-23) = 1+2^-8+2^-31-2^-46: the float32 product rounds
    # onto the bf16 tie 1+2^-8, which then rounds to even 0x3F80 (a single
    # rounding of the exact product would give 0x3F81)
    assert bits[1, 64] == 0x3F80
    # zero level decodes to +0, never -0
    assert bits[0, 2] == 0 and bits[0, 100] == 0
    vals = oracle.decode_q4(packed, absmax, cb, n, k)
    assert vals[0, 0] == 2.0 and vals[1, 1] == 0.1875


def test_q4_extremes_decode_to_absmax():
    cb = np.linspace(-1, 1, 16).astype(np.float32)
    g = np.random.default_rng(8)
    am = np.abs(g.standard_normal(4).astype(np.float32))
    codes = np.zeros((1, 256), np.uint8); codes[0, 1::2] = 15
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    bits = oracle.decode_q4_bits(packed, am, cb, 1, 256)
    exp_neg = bf16_bits_of(to_bf16_values(-np.repeat(am, 64)))
    exp_pos = bf16_bits_of(to_bf16_values(np.repeat(am, 64)))
    assert np.array_equal(bits[0, 0::2], exp_neg[0::2])
    assert np.array_equal(bits[0, 1::2], exp_pos[1::2])


def test_config_inputs_roundtrip_through_oracle_shapes():
    li = gen_linear(16, 64, 32, 4, 16.0, "bf16")
    Y = oracle.linear_fwd(li.X, li.W, li.A, li.B, oracle.scaling(li.alpha, li.r))
    assert Y.shape == (16, 32) and np.isfinite(Y).all()
    mi = gen_mlp(8, 64, 128, 4, 16.0, "bf16")
    Y, e, g = oracle.mlp_fwd(mi.X, mi.W, mi.A, mi.B, 4.0)
    assert Y.shape == (8, 64) and e.shape == (8, 128)


# ------------------------------------------- double-quantised block constants
def _f32(v):
    return np.float32(v)


def test_absmax_dq_hand_fixture():
    # levels, scales and offset chosen so that every value is worked out by hand
    table = np.zeros(256, np.float32)
    table[0], table[255], table[128], table[7] = -1.0, 1.0, 0.5, 0.125
    scale = np.array([0.25, 2.0], np.float32)
    codes8 = np.full(300, 7, np.uint8)            # 0.125 everywhere else
    codes8[[0, 1, 255, 256, 299]] = [255, 0, 128, 128, 0]
    am = oracle.decode_absmax_dq(codes8, table, scale, 0.5, 300)
    assert am.dtype == np.float32 and am.shape == (300,)
    assert am[0] == 0.75          # 1 * 0.25 + 0.5
    assert am[1] == 0.25          # -1 * 0.25 + 0.5
    assert am[2] == 0.53125       # 0.125 * 0.25 + 0.5
    assert am[255] == 0.625       # last block of the first 256-group: scale[0]
    assert am[256] == 1.5         # first block of the second group: scale[1]
    assert am[257] == 0.75        # 0.125 * 2 + 0.5
    assert am[299] == -1.5        # -1 * 2 + 0.5
    with pytest.raises(ValueError):
        oracle.decode_absmax_dq(codes8, table, scale[:1], 0.5, 300)   # group 1 has no scale


def test_absmax_dq_rounds_product_then_sum():
    # (1+2^-12)^2 = 1 + 2^-11 + 2^-24: the float32 product rounds the 2^-24
    # tie to even (1 + 2^-11); adding -1 then gives exactly 2^-11.  A fused
    # multiply-add would keep the 2^-24 and give 2^-11 + 2^-24.
    t = np.zeros(256, np.float32)
    t[9] = 1 + 2**-12
    am = oracle.decode_absmax_dq(np.array([9], np.uint8), t, np.array([1 + 2**-12], np.float32),
                                 -1.0, 1)
    assert am[0] == _f32(2**-11)
    assert am[0] != _f32(2**-11 + 2**-24)
    # the sum rounds too: 1 + 2^-24 is a tie -> 1.0 (even); 1 + 3*2^-24 is a
    # tie between 1 + 2^-23 (odd) and 1 + 2^-22 (even) -> 1 + 2^-22
    t[9] = 1.0
    one = np.array([1.0], np.float32)
    assert oracle.decode_absmax_dq(np.array([9], np.uint8), t, one, 2**-24, 1)[0] == 1.0
    assert oracle.decode_absmax_dq(np.array([9], np.uint8), t, one, 3 * 2**-24, 1)[0] == \
        _f32(1 + 2**-22)


def test_q4dq_decode_is_q4_decode_with_the_constants():
    # the hand-fixture constants above, written out, drive the plain decode
    table = np.zeros(256, np.float32)
    table[0], table[255], table[128], table[7] = -1.0, 1.0, 0.5, 0.125
    scale = np.array([0.25, 2.0], np.float32)
    n, k = 4, 64 * 75                              # 300 blocks
    codes8 = np.full(300, 7, np.uint8)
    codes8[[0, 1, 255, 256, 299]] = [255, 0, 128, 128, 0]
    am = np.full(300, 0.53125, np.float32)
    am[256:] = 0.75
    am[[0, 1, 255, 256, 299]] = [0.75, 0.25, 0.625, 1.5, -1.5]
    g = np.random.default_rng(5)
    codes = g.integers(0, 16, size=(n, k), dtype=np.uint8)
    packed = (codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8)
    cb = make_codebook()
    got = oracle.decode_q4dq_bits(packed, codes8, table, scale, 0.5, cb, n, k)
    assert np.array_equal(got, oracle.decode_q4_bits(packed, am, cb, n, k))


def test_absmax_dq_elementwise_loop():
    # per-element loop: the product of two float32 is exact in a Python
    # float; np.float32() rounds it to nearest even; with every term within
    # 2^-16 .. 1 the float sum is exact again before its own rounding
    g = np.random.default_rng(11)
    nblk = 700
    c8 = g.integers(0, 256, size=nblk, dtype=np.uint8)
    table = make_absmax_codebook()
    scale = g.uniform(0.01, 0.03, size=3).astype(np.float32)
    off = np.float32(0.04)
    want = np.empty(nblk, np.float32)
    for b in range(nblk):
        m = np.float32(float(table[int(c8[b])]) * float(scale[b // 256]))
        want[b] = np.float32(float(m) + float(off))
    got = oracle.decode_absmax_dq(c8, table, scale, off, nblk)
    assert np.array_equal(got.view(np.uint32), want.view(np.uint32))
    assert (got > 0).all()


def test_generated_dq_weight_layout():
    li = gen_linear(4, 128, 72, 4, 16.0, "bf16", seed=3, q4="dq")
    q = li.q4
    assert q.absmax is None and q.double_quant
    nblk = 72 * 128 // 64
    assert q.absmax_codes.shape == (nblk,) and q.absmax_codes.dtype == np.uint8
    assert q.absmax_scale.shape == ((nblk + 255) // 256,)
    assert q.absmax_codebook.shape == (256,) and q.absmax_blocksize == 256
    W = oracle.decode_q4_weight(q)
    assert W.shape == (72, 128) and np.isfinite(W).all()
    assert np.abs(W).max() <= 0.07


# ------------------------------------------------------------------ RMSNorm
def test_rmsnorm_constant_rows_closed_form():
    # a row of equal values c: mean of squares c^2, so Y = c / sqrt(c^2 + eps) w
    w = np.array([1.0, -2.0, 0.5, 3.0])
    X = np.array([[2.0] * 4, [-0.5] * 4, [0.0] * 4])
    Y, rstd = oracle.rmsnorm_fwd(X, w, 0.25)
    assert np.allclose(rstd, [1 / math.sqrt(4.25), 1 / math.sqrt(0.5), 2.0], rtol=1e-15)
    assert np.allclose(Y[0], 2.0 / math.sqrt(4.25) * w, rtol=1e-15)
    assert np.allclose(Y[1], -0.5 / math.sqrt(0.5) * w, rtol=1e-15)
    assert np.all(Y[2] == 0.0)
    # eps = 0: a constant row normalises to sign(c) w
    Y0, _ = oracle.rmsnorm_fwd(X[:2], w, 0.0)
    assert np.allclose(Y0, [w, -w], rtol=1e-15)


def test_rmsnorm_hand_row():
    # X = [3, 4]: mean of squares 12.5, eps 0.0 -> rstd = 1/sqrt(12.5)
    Y, rstd = oracle.rmsnorm_fwd(np.array([[3.0, 4.0]]), np.array([1.0, 10.0]), 0.0)
    assert abs(rstd[0] - 1 / math.sqrt(12.5)) < 1e-16
    assert np.allclose(Y[0], [3 / math.sqrt(12.5), 40 / math.sqrt(12.5)], rtol=1e-15)
    # unit root-mean-square rows pass through unchanged (times w)
    X = np.array([[1.0, -1.0, 1.0, -1.0]])
    assert np.allclose(oracle.rmsnorm_fwd(X, np.ones(4), 0.0)[0], X, rtol=1e-15)


def test_rmsnorm_scale_invariance_and_orthogonal_gradient():
    g = np.random.default_rng(3)
    X, w, dY = g.standard_normal((5, 12)), g.standard_normal(12), g.standard_normal((5, 12))
    Y, _ = oracle.rmsnorm_fwd(X, w, 0.0)
    Y3, _ = oracle.rmsnorm_fwd(3.5 * X, w, 0.0)
    assert np.allclose(Y, Y3, rtol=1e-13)
    # with eps = 0 the output does not change along x, so the gradient is
    # orthogonal to x row by row
    dX = oracle.rmsnorm_bwd(X, w, 0.0, dY)
    assert np.allclose(np.sum(dX * X, axis=1), 0.0, atol=1e-12)


def test_rmsnorm_gradient_finite_differences():
    g = np.random.default_rng(4)
    X, w, dY = g.standard_normal((3, 7)), g.standard_normal(7), g.standard_normal((3, 7))
    eps = 1e-2
    loss = lambda: float(np.sum(dY * oracle.rmsnorm_fwd(X, w, eps)[0]))
    assert oracle.rel_fro(oracle.rmsnorm_bwd(X, w, eps, dY), _fd(loss, X)) < 1e-7


def test_rmsnorm_against_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    g = np.random.default_rng(6)
    X, w, dY = g.standard_normal((9, 16)), g.standard_normal(16), g.standard_normal((9, 16))
    eps = 1e-5
    tX = torch.tensor(X, requires_grad=True)
    ty = tX * torch.rsqrt(tX.pow(2).mean(-1, keepdim=True) + eps) * torch.tensor(w)
    ty.backward(torch.tensor(dY))
    Y, _ = oracle.rmsnorm_fwd(X, w, eps)
    assert np.allclose(Y, ty.detach().numpy(), rtol=1e-13, atol=1e-15)
    assert np.allclose(oracle.rmsnorm_bwd(X, w, eps, dY), tX.grad.numpy(), rtol=1e-12,
                       atol=1e-14)


# ------------------------------------------------------- comparator, dispatch
def test_rel_fro_hand_cases():
    # ||x - ref||_F / ||ref||_F worked out by hand
    x = np.array([3.0, 4.0])
    assert oracle.rel_fro(x, x) == 0.0
    assert oracle.rel_fro(np.zeros(2), np.zeros(2)) == 0.0              # both zero
    assert oracle.rel_fro(x, np.zeros(2)) == math.inf                   # zero reference
    assert oracle.rel_fro(np.zeros(2), x) == 1.0                        # zero result
    assert oracle.rel_fro(-x, x) == 2.0                                 # sign flip: ||2x||/||x||
    assert oracle.rel_fro(x + np.array([0.5, 0.0]), x) == 0.1           # |delta| / ||x|| = 0.5 / 5
    # both components off by one: sqrt(2) / 5 (a max-abs or squared-norm
    # comparator gives 0.2 or 0.08 here)
    assert abs(oracle.rel_fro(np.array([4.0, 5.0]), x) - math.sqrt(2.0) / 5.0) < 1e-15
    # matrices are compared element by element over the whole tensor:
    # diff [[0, 2], [2, 0]] has norm sqrt(8), the identity sqrt(2)
    got = oracle.rel_fro(np.array([[1.0, 2.0], [2.0, 1.0]]), np.eye(2))
    assert abs(got - 2.0) < 1e-15
    # a permutation with the same norm is far off, not equal
    assert oracle.rel_fro(x[::-1].copy(), x) == math.sqrt(2.0) / 5.0
    # not symmetric: the reference's norm is the denominator
    assert abs(oracle.rel_fro(np.array([6.0, 8.0]), x) - 1.0) < 1e-15
    assert abs(oracle.rel_fro(x, np.array([6.0, 8.0])) - 0.5) < 1e-15
    # float32 inputs are compared in float64 (no float32 cancellation)
    a = np.array([1.0 + 2**-20], dtype=np.float32)
    assert abs(oracle.rel_fro(a, np.array([1.0], dtype=np.float32)) - 2**-20) < 1e-18


def test_decode_q4_weight_dispatches_on_container_form():
    # plain block constants, hand-worked: n = 2 rows of k = 64, codes 0x21
    # (element 2j -> level 1, element 2j+1 -> level 2), row 0 scale 2, row 1 0.5
    from types import SimpleNamespace
    cb = np.array([0.0, 0.25, -0.5] + [0.0] * 13, dtype=np.float32)
    codes = np.full((2, 32), 0x21, dtype=np.uint8)
    q = SimpleNamespace(codes=codes, absmax=np.array([2.0, 0.5], np.float32), codebook=cb,
                        n=2, k=64, blocksize=64, absmax_codes=None)
    W = oracle.decode_q4_weight(q)
    assert W.shape == (2, 64)
    assert (W[0, 0::2] == 0.5).all() and (W[0, 1::2] == -1.0).all()
    assert (W[1, 0::2] == 0.125).all() and (W[1, 1::2] == -0.25).all()
    # double-quantised constants, hand-worked: table[c] * scale + offset
    # block 0: 0.5 * 2 + 1 = 2;  block 1: 0.25 * 2 + 1 = 1.5
    table = np.zeros(256, np.float32); table[7] = 0.5; table[9] = 0.25
    qd = SimpleNamespace(codes=codes, absmax=None, codebook=cb, n=2, k=64, blocksize=64,
                         absmax_codes=np.array([7, 9], np.uint8), absmax_codebook=table,
                         absmax_scale=np.array([2.0], np.float32), absmax_offset=1.0,
                         absmax_blocksize=256)
    Wd = oracle.decode_q4_weight(qd)
    assert Wd.shape == (2, 64)
    assert (Wd[0, 0::2] == 0.5).all() and (Wd[0, 1::2] == -1.0).all()
    assert (Wd[1, 0::2] == 0.375).all() and (Wd[1, 1::2] == -0.75).all()
    # a generated container of each form decodes to the bits of its own
    # branch: non-square (n != k) and several 64-blocks per row
    for kind in ("plain", "dq"):
        li = gen_linear(4, 128, 72, 4, 16.0, "bf16", seed=5, q4=kind if kind == "dq" else True)
        qq = li.q4
        if kind == "dq":
            bits = oracle.decode_q4dq_bits(qq.codes, qq.absmax_codes, qq.absmax_codebook,
                                           qq.absmax_scale, qq.absmax_offset, qq.codebook,
                                           72, 128)
        else:
            bits = oracle.decode_q4_bits(qq.codes, qq.absmax, qq.codebook, 72, 128)
        got = oracle.decode_q4_weight(qq)
        assert got.shape == (72, 128)
        assert np.array_equal(bf16_bits_of(got), bits)
