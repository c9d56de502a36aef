"""Seeded synthetic inputs for the LoRA linear layer and the LoRA-SwiGLU MLP.

This module is shared by the CPU oracle (tests, bench baseline) and the GPU
path.  It holds none of the method's arithmetic: it only draws random tensors,
rounds them to their storage dtype, packs 4-bit codes and builds the 16-level
codebook *data*.  Every function returns float32 numpy arrays whose values are
exactly representable in the storage dtype (bf16 or fp32), so the oracle can
upcast them to float64 exactly and the GPU can downcast them to bf16 exactly.

Workload recipes (shapes and distributions) follow the five configurations of
the benchmark: X, dY ~ N(0,1); W ~ N(0,0.02); A ~ U(+-1/sqrt(in_features)) (the
bound of Kaiming-uniform with a=sqrt(5) that the LoRA reference layer of the
"Unsloth deep-dive" page (chenxutan.com/d/6058, section 1.3) applies to A);
B ~ N(0, b_std) with b_std = 0.02 (B != 0 on purpose, so the adapter term is
exercised; B = 0 is the page's initialisation and is used by invariant tests).
The 4-bit workload draws codes uniformly over 0..15 and one fp32 absmax
~ |N(0,0.05)| per block of 64 consecutive in-features of a weight row.  The
double-quantised 4-bit form (q4="dq") draws the blocks' 8-bit constant codes
uniformly over 0..255, one scale ~ U(0.01, 0.03) per 256 blocks and uses the
offset 0.04 with a 256-level table evenly spaced over [-1, 1].
"""
from __future__ import annotations

import math
from dataclasses import dataclass, field
from typing import Dict, Optional

import numpy as np

BASE_SEED = 3407          # the pages' random_state / seed value
Q4_BLOCK = 64


# --------------------------------------------------------------------------
# storage-dtype rounding (library routine, not the method's arithmetic)
# --------------------------------------------------------------------------
def to_bf16_values(x: np.ndarray) -> np.ndarray:
    """Round float32 values to the nearest bf16 (torch's conversion) and
    return them as float32 (exact images of the bf16 values)."""
    import torch
    t = torch.from_numpy(np.ascontiguousarray(x, dtype=np.float32))
    return t.to(torch.bfloat16).to(torch.float32).numpy()


def bf16_bits_of(x: np.ndarray) -> np.ndarray:
    """uint16 bit patterns of float32 values that are exactly bf16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32)
    return (u >> 16).astype(np.uint16)


# --------------------------------------------------------------------------
# 16-level signed normal-quantile codebook (data for the 4-bit format)
# --------------------------------------------------------------------------
def make_codebook() -> np.ndarray:
    """16 float32 levels in [-1, 1], sorted ascending, containing -1, 0, +1.

    Levels are quantiles of the standard normal distribution: 8 positive
    levels at evenly spaced probabilities in (0.5, p_max], 7 negative levels
    mirrored at evenly spaced probabilities, each side normalised so its
    extreme level is exactly +-1, plus an exact zero (the asymmetric 4-bit
    NormalFloat construction that the pages name but do not tabulate).
    """
    from scipy.special import ndtri
    p_max = 0.5 * ((1.0 - 1.0 / 32.0) + (1.0 - 1.0 / 30.0))
    pos = ndtri(np.linspace(p_max, 0.5, 9)[:-1])        # 8 values > 0
    neg = -ndtri(np.linspace(p_max, 0.5, 8)[:-1])       # 7 values < 0
    pos = pos / pos.max()
    neg = neg / (-neg.min())
    levels = np.concatenate([pos, [0.0], neg]).astype(np.float64)
    levels = np.sort(levels).astype(np.float32)
    levels[0] = -1.0
    levels[-1] = 1.0
    return levels


# --------------------------------------------------------------------------
# tensor containers
# --------------------------------------------------------------------------
def make_absmax_codebook() -> np.ndarray:
    """256 float32 levels evenly spaced over [-1, 1] (level c = (2c - 255) /
    255): the table the 8-bit codes of double-quantised block constants
    index in the synthetic weights."""
    c = np.arange(256, dtype=np.float64)
    return ((2.0 * c - 255.0) / 255.0).astype(np.float32)


@dataclass
class Q4Weight:
    """4-bit base weight [n x k]: codes[n, k/2] (flat element 2j in the low
    nibble of byte j), absmax[n*k/64] fp32 (block = 64 consecutive k of one
    row), codebook[16] fp32.

    Double-quantised form (absmax None): absmax_codes[n*k/64] uint8,
    absmax_codebook[256] fp32, absmax_scale[ceil(n*k/64 / 256)] fp32 and
    one float absmax_offset."""
    n: int
    k: int
    codes: np.ndarray
    absmax: Optional[np.ndarray]
    codebook: np.ndarray
    blocksize: int = Q4_BLOCK
    absmax_codes: Optional[np.ndarray] = None
    absmax_codebook: Optional[np.ndarray] = None
    absmax_scale: Optional[np.ndarray] = None
    absmax_offset: float = 0.0
    absmax_blocksize: int = 256

    @property
    def double_quant(self) -> bool:
        return self.absmax_codes is not None


@dataclass
class LinearInputs:
    dtype: str                 # "f32" or "bf16"
    T: int
    k: int
    n: int
    r: int
    alpha: float
    X: np.ndarray              # [T, k]
    W: Optional[np.ndarray]    # [n, k] (None when q4 is set)
    A: np.ndarray              # [r, k]
    B: np.ndarray              # [n, r]
    dY: np.ndarray             # [T, n]
    q4: Optional[Q4Weight] = None


@dataclass
class MLPInputs:
    dtype: str
    T: int
    d: int
    f: int
    r: int
    alpha: float
    X: np.ndarray              # [T, d]
    W: Dict[str, Optional[np.ndarray]]   # "gate","up": [f, d]; "down": [d, f]
    A: Dict[str, np.ndarray]   # gate/up: [r, d]; down: [r, f]
    B: Dict[str, np.ndarray]   # gate/up: [f, r]; down: [d, r]
    dY: np.ndarray             # [T, d]
    q4: Dict[str, Q4Weight] = field(default_factory=dict)


def _rngs(seed: int, count: int):
    return [np.random.Generator(np.random.PCG64(s))
            for s in np.random.SeedSequence(seed).spawn(count)]


def _normal(rng, shape, std, dtype):
    x = rng.standard_normal(size=shape, dtype=np.float32)
    if std != 1.0:
        x *= np.float32(std)
    return to_bf16_values(x) if dtype == "bf16" else x


def _uniform(rng, shape, bound, dtype):
    x = rng.uniform(-bound, bound, size=shape).astype(np.float32)
    return to_bf16_values(x) if dtype == "bf16" else x


def _q4(rng, n, k, codebook, dq=False) -> Q4Weight:
    """Random 4-bit codes; block constants drawn directly (plain: |N(0,
    0.05^2)|; double-quantised: uniform 8-bit codes, per-256-block scales
    uniform in [0.01, 0.03], offset 0.04, so every constant lies in (0,
    0.07]).  Nothing is quantised here: the codes are the data."""
    if k % Q4_BLOCK:
        raise ValueError("4-bit weights need k % 64 == 0")
    codes = rng.integers(0, 16, size=(n, k), dtype=np.uint8)
    packed = np.ascontiguousarray((codes[:, 0::2] | (codes[:, 1::2] << 4)).astype(np.uint8))
    nblk = (n * k) // Q4_BLOCK
    if dq:
        acodes = rng.integers(0, 256, size=nblk, dtype=np.uint8)
        scale = rng.uniform(0.01, 0.03, size=(nblk + 255) // 256).astype(np.float32)
        return Q4Weight(n, k, packed, None, codebook.copy(), Q4_BLOCK, acodes,
                        make_absmax_codebook(), scale, 0.04)
    absmax = np.abs(rng.standard_normal(size=nblk, dtype=np.float32) * np.float32(0.05))
    return Q4Weight(n, k, packed, absmax.astype(np.float32), codebook.copy())


def gen_linear(T, k, n, r, alpha, dtype="bf16", seed=BASE_SEED, b_std=0.02,
               w_std=0.02, q4=False, X=None) -> LinearInputs:
    """One LoRA linear layer's tensors; pass X to share an input tensor."""
    rx, rw, ra, rb, rdy = _rngs(seed, 5)
    X = _normal(rx, (T, k), 1.0, dtype) if X is None else X
    qw = None
    W = None
    if q4:
        qw = _q4(rw, n, k, make_codebook(), dq=(q4 == "dq"))
    else:
        W = _normal(rw, (n, k), w_std, dtype)
    A = _uniform(ra, (r, k), 1.0 / math.sqrt(k), dtype)
    B = _normal(rb, (n, r), b_std, dtype)
    dY = _normal(rdy, (T, n), 1.0, dtype)
    return LinearInputs(dtype, T, k, n, r, float(alpha), X, W, A, B, dY, qw)


def gen_mlp(T, d, f, r, alpha, dtype="bf16", seed=BASE_SEED, b_std=0.02,
            w_std=0.02, q4=False) -> MLPInputs:
    rng = _rngs(seed, 11)
    X = _normal(rng[0], (T, d), 1.0, dtype)
    shapes = {"gate": (f, d), "up": (f, d), "down": (d, f)}
    W, A, B, Q = {}, {}, {}, {}
    cb = make_codebook()
    for i, name in enumerate(("gate", "up", "down")):
        n_out, k_in = shapes[name]
        if q4:
            Q[name] = _q4(rng[1 + 3 * i], n_out, k_in, cb, dq=(q4 == "dq"))
            W[name] = None
        else:
            W[name] = _normal(rng[1 + 3 * i], (n_out, k_in), w_std, dtype)
        A[name] = _uniform(rng[2 + 3 * i], (r, k_in), 1.0 / math.sqrt(k_in), dtype)
        B[name] = _normal(rng[3 + 3 * i], (n_out, r), b_std, dtype)
    dY = _normal(rng[10], (T, d), 1.0, dtype)
    return MLPInputs(dtype, T, d, f, r, float(alpha), X, W, A, B, dY, Q)


@dataclass
class RMSNormInputs:
    dtype: str
    T: int
    d: int
    eps: float
    X: np.ndarray              # [T, d] the residual stream in front of the norm
    w: np.ndarray              # [d] norm weight
    dY: np.ndarray             # [T, d] upstream gradient of the normalised rows


def gen_rmsnorm(T, d, dtype="bf16", seed=BASE_SEED, eps=1e-5, x_std=1.0) -> RMSNormInputs:
    """X ~ N(0, x_std^2), w ~ 1 + N(0, 0.1^2) (a trained norm weight near its
    initial value 1), dY ~ N(0, 1); eps 1e-5."""
    rx, rw, rdy = _rngs(seed, 3)
    X = _normal(rx, (T, d), x_std, dtype)
    w = rw.standard_normal(size=d, dtype=np.float32) * np.float32(0.1) + np.float32(1.0)
    w = to_bf16_values(w) if dtype == "bf16" else w.astype(np.float32)
    dY = _normal(rdy, (T, d), 1.0, dtype)
    return RMSNormInputs(dtype, T, d, float(eps), X, w, dY)


# --------------------------------------------------------------------------
# the five benchmark workloads
# --------------------------------------------------------------------------
CONFIGS = {
    1: dict(kind="linear", dtype="f32", T=256, k=512, n=512, r=8, alpha=16.0),
    2: dict(kind="mlp", dtype="bf16", T=8192, d=2048, f=8192, r=16, alpha=16.0),
    3: dict(kind="mlp", dtype="bf16", T=8192, d=4096, f=14336, r=16, alpha=16.0),
    4: dict(kind="attn_mlp", dtype="bf16", T=16384, d=4096, f=14336, d_kv=1024,
            r=64, alpha=16.0),
    5: dict(kind="mlp", dtype="bf16", T=8192, d=4096, f=14336, r=16, alpha=16.0,
            q4=True),
}


def gen_config(cfg: int, seed: Optional[int] = None, b_std=0.02, scale_T=None, part=None,
               q4=None):
    """Inputs of one benchmark workload.  `scale_T` optionally replaces T
    (same distributions, fewer tokens) for bounded samples.  For workload 4,
    `part` = "attn" or "mlp" generates only that half.  `q4` (MLP workloads)
    overrides the base-weight form: False, True (4-bit) or "dq" (4-bit with
    double-quantised block constants)."""
    c = dict(CONFIGS[cfg])
    if q4 is not None:
        c["q4"] = q4
    seed = BASE_SEED + cfg if seed is None else seed
    T = c["T"] if scale_T is None else scale_T
    if c["kind"] == "linear":
        return gen_linear(T, c["k"], c["n"], c["r"], c["alpha"], c["dtype"], seed,
                          b_std=b_std)
    if c["kind"] == "mlp":
        return gen_mlp(T, c["d"], c["f"], c["r"], c["alpha"], c["dtype"], seed,
                       b_std=b_std, q4=c.get("q4", False))
    # attention projections + MLP: q/k/v share X_attn, o has its own input
    d, dkv = c["d"], c["d_kv"]
    out = {}
    if part in (None, "attn"):
        layers = {}
        layers["q"] = gen_linear(T, d, d, c["r"], c["alpha"], "bf16", seed * 10 + 1, b_std)
        Xq = layers["q"].X
        layers["k"] = gen_linear(T, d, dkv, c["r"], c["alpha"], "bf16", seed * 10 + 2, b_std, X=Xq)
        layers["v"] = gen_linear(T, d, dkv, c["r"], c["alpha"], "bf16", seed * 10 + 3, b_std, X=Xq)
        layers["o"] = gen_linear(T, d, d, c["r"], c["alpha"], "bf16", seed * 10 + 4, b_std)
        out["attn"] = layers
    if part in (None, "mlp"):
        out["mlp"] = gen_mlp(T, d, c["f"], c["r"], c["alpha"], "bf16", seed * 10 + 5, b_std)
    return out
