"""CPU oracle for the LoRA linear layer and the LoRA-SwiGLU MLP (test infrastructure).

THIS MODULE IS TEST INFRASTRUCTURE.  Only the test suite, the package smoke
check and the benchmark's CPU-baseline leg may import it.  The GPU library
never calls it and shares no code with it.

Everything is evaluated in float64 on the exact float64 images of the inputs
(fp32 values, or bf16 values for the bf16 workloads), with no intermediate
rounding.  The one place where rounding is part of the definition is the
4-bit decode, which produces bf16 weights; it is written out bit by bit.

Sources (web pages; sections as printed on them):
  [DD]  "Unsloth deep-dive: Triton kernels + hand-written backprop"
        (chenxutan.com/d/6058): 1.2 low-rank update, 1.3 init and the
        LoRALayer / LinearWithLoRA reference code, 1.4 QLoRA/NF4,
        2.4 hand-written backward.
  [WHY] "Why Unsloth trains 5-8x faster" (mokono.cn/news/868259):
        3.1-3.2 fused LoRA kernel, 5.2 fused 4-bit dequant + matmul.
  [CR]  "Unsloth code-reading guide" (ai-reference-codex.pages.dev/
        frontier/unsloth): 2.1 4-bit weights decoded to bf16 every step,
        2.3 manual LoRA path, 4 LoRA_MLP saves only X, e, g.
  [TB] "Unsloth speed secrets: Triton kernels accelerate backprop"
        (mokono.cn/news/201055): 3.2 RMSNorm kernel.
  [HF]  "Unsloth + TRL compiled blog" (bbs.huaweicloud.com/blogs/510494),
        section 1: SwiGLU named as a fused activation.

Pins (tests/test_oracle_pins.py): printed trainable-parameter count, B = 0
invariant, merged-weight invariant, brute-force loops on tiny shapes, central
finite differences of every gradient, torch.autograd in float64, silu closed
forms, bf16 rounding against torch, hand-computed 4-bit decodes, and
hand-computed double-quantised block constants (including a case where a
fused multiply-add would round differently) plus a per-element loop, the
comparator rel_fro on hand-worked vectors and matrices (zero reference, sign
flip, one-component and all-component errors, asymmetry), and the 4-bit
container dispatch on hand-worked containers of both forms.
tests/test_oracle_mutants.py plants 39 single-expression slips in a copy of
this module (dropped terms and scales, wrong signs, a transposed operand,
wrong indices, nibble order and rounding mode, a comparator that takes a
difference of norms, a max-abs, a squared or an unnormalised error) and
checks that each one fails at least one of those pins.
"""
from __future__ import annotations

import numpy as np

F64 = np.float64


def _f64(x):
    return np.asarray(x, dtype=F64)


# ---------------------------------------------------------------------------
# LoRA linear layer
# ---------------------------------------------------------------------------
def scaling(alpha: float, r: int) -> float:
    """s = alpha / rank  ([DD] 1.3, the LoRALayer's `scaling` attribute)."""
    return float(alpha) / float(r)


def trainable_params(n: int, k: int, r: int) -> int:
    """Adapter parameter count r*(n+k) for a frozen n x k weight ([DD] 1.2)."""
    return r * n + r * k


def merged_weight(W, A, B, s):
    """W' = W + s * B.A: the low-rank update added to the frozen weight
    ([DD] 1.2, delta W = B.A; the page's merged-16bit export, section 5.1)."""
    return _f64(W) + s * (_f64(B) @ _f64(A))


def linear_fwd(X, W, A, B, s):
    """Y = X W^T + s (X A^T) B^T.

    [DD] 1.3: the layer's output is the frozen base linear plus the LoRA
    branch `x @ A.T @ B.T * scaling` (dropout = identity: the workloads have
    none, and the guide [CR] 5 says the fast path requires dropout 0 and no
    bias).  A is [r x in], B is [out x r] as in the page's code.
    """
    X, W, A, B = map(_f64, (X, W, A, B))
    H = X @ A.T                       # the rank-r product x_a ([WHY] 3.1)
    return X @ W.T + s * (H @ B.T)


def linear_bwd(X, W, A, B, s, dY, want_dx=True):
    """Closed-form gradients of the LoRA linear layer; W is frozen (no dW).

    With H = X A^T and G = dY B (chain rule through Y = X W^T + s H B^T):
      dX = dY W + s G A,   dA = s G^T X,   dB = s dY^T H.
    [DD] 2.4 and [CR] 2.3/4: gradients are written from derived formulas
    instead of an autograd graph; the base weight has requires_grad=False.
    """
    X, W, A, B, dY = map(_f64, (X, W, A, B, dY))
    G = dY @ B
    H = X @ A.T
    dX = dY @ W + s * (G @ A) if want_dx else None
    dA = s * (G.T @ X)
    dB = s * (dY.T @ H)
    return dX, dA, dB


# ---------------------------------------------------------------------------
# SwiGLU
# ---------------------------------------------------------------------------
def sigmoid(z):
    """logistic function 1/(1+exp(-z)) in float64."""
    z = _f64(z)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-z))


def swiglu(e, g):
    """h = silu(e) * g, silu(z) = z * sigmoid(z): the gated activation of the
    SwiGLU MLP ([HF] 1, [CR] 7 swiglu_fg_kernel), gate e, up g."""
    e, g = _f64(e), _f64(g)
    return e * sigmoid(e) * g


def swiglu_bwd(e, g, dh):
    """Derivative of h = e sigmoid(e) g, recomputed from the saved e, g:
      dh/de = g * sigmoid(e) * (1 + e (1 - sigmoid(e))),  dh/dg = e sigmoid(e).
    ([CR] 4: LoRA_MLP saves only X, e, g; the backward recomputes the rest.)"""
    e, g, dh = _f64(e), _f64(g), _f64(dh)
    sg = sigmoid(e)
    de = dh * g * sg * (1.0 + e * (1.0 - sg))
    dg = dh * e * sg
    return de, dg


# ---------------------------------------------------------------------------
# LoRA-SwiGLU MLP (three LoRA linears: gate, up, down)
# ---------------------------------------------------------------------------
def mlp_fwd(X, W, A, B, s):
    """e = lin(X; gate), g = lin(X; up), h = silu(e) g, Y = lin(h; down).
    W, A, B are dicts keyed "gate", "up", "down".  Returns (Y, e, g): the MLP
    saves X, e, g for the backward ([CR] 2.3 apply_lora_mlp_swiglu, 4)."""
    e = linear_fwd(X, W["gate"], A["gate"], B["gate"], s)
    g = linear_fwd(X, W["up"], A["up"], B["up"], s)
    h = swiglu(e, g)
    Y = linear_fwd(h, W["down"], A["down"], B["down"], s)
    return Y, e, g


def mlp_bwd(X, W, A, B, s, dY, want_dx=True):
    """Closed-form MLP backward from X (e, g recomputed in float64).

    down:      (dh, dA_d, dB_d) = linear_bwd(h, dY; down)
    SwiGLU:    (de, dg) = swiglu_bwd(e, g, dh)
    gate, up:  (dX_g, dA_g, dB_g) = linear_bwd(X, de; gate), same for up
    dX = dX_g + dX_u (both projections read the same X).
    Returns dict with dX (or None) and dA_*/dB_* per projection.
    """
    e = linear_fwd(X, W["gate"], A["gate"], B["gate"], s)
    g = linear_fwd(X, W["up"], A["up"], B["up"], s)
    h = swiglu(e, g)
    dh, dAd, dBd = linear_bwd(h, W["down"], A["down"], B["down"], s, dY)
    de, dg = swiglu_bwd(e, g, dh)
    dXg, dAg, dBg = linear_bwd(X, W["gate"], A["gate"], B["gate"], s, de, want_dx)
    dXu, dAu, dBu = linear_bwd(X, W["up"], A["up"], B["up"], s, dg, want_dx)
    out = {"dA_gate": dAg, "dB_gate": dBg, "dA_up": dAu, "dB_up": dBu,
           "dA_down": dAd, "dB_down": dBd, "dX": None}
    if want_dx:
        out["dX"] = dXg + dXu
    return out


# ---------------------------------------------------------------------------
# bf16 rounding and the 4-bit decode
# ---------------------------------------------------------------------------
def bf16_rne_bits(x32) -> np.ndarray:
    """Round float32 values to bf16 with round-to-nearest-even, on the bit
    patterns (integer arithmetic); returns uint16.  NaN stays NaN (quiet),
    +-inf and +-0 are kept."""
    u = np.ascontiguousarray(x32, dtype=np.float32).view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    rounded = (u + 0x7FFF + lsb) >> 16
    is_nan = ((u & 0x7F800000) == 0x7F800000) & ((u & 0x007FFFFF) != 0)
    out = np.where(is_nan, (u >> 16) | 0x40, rounded)
    return out.astype(np.uint16)


def bf16_bits_to_f64(bits) -> np.ndarray:
    b = np.asarray(bits, dtype=np.uint16).astype(np.uint32) << 16
    return b.view(np.float32).astype(F64)


def decode_q4_bits(codes, absmax, codebook, n, k, blocksize=64) -> np.ndarray:
    """Decode a 4-bit weight [n x k] to bf16 bit patterns.

    For flat row-major index i:  byte = codes[i // 2]; c = low nibble if i
    is even else high nibble; w32 = codebook[c] * absmax[i // blocksize]
    (one IEEE float32 multiply, round to nearest even); W[i] = bf16(w32)
    with round-to-nearest-even.
    ([DD] 1.4 NF4 codes with per-block constants; [CR] 2.1 the 4-bit weights
    are dequantised to bf16 before every matmul; [WHY] 5.2 the decode is
    fused with the matmul, which must not change the decoded values.)
    """
    if blocksize != 64 or (n * k) % blocksize or k % 2:
        raise ValueError("unsupported 4-bit layout")
    flat = np.asarray(codes, dtype=np.uint8).reshape(-1)
    nib = np.empty(n * k, dtype=np.uint8)
    nib[0::2] = flat & 0x0F
    nib[1::2] = flat >> 4
    cb = np.asarray(codebook, dtype=np.float32)
    am = np.asarray(absmax, dtype=np.float32).reshape(-1)
    w32 = cb[nib] * np.repeat(am, blocksize)          # float32 * float32 -> float32
    return bf16_rne_bits(w32.astype(np.float32)).reshape(n, k)


def decode_q4(codes, absmax, codebook, n, k, blocksize=64) -> np.ndarray:
    """Decoded 4-bit weight as float64 values (exact images of the bf16s)."""
    return bf16_bits_to_f64(decode_q4_bits(codes, absmax, codebook, n, k, blocksize))


def decode_absmax_dq(absmax_codes, absmax_codebook, absmax_scale, absmax_offset,
                     nblocks, blocksize2=256) -> np.ndarray:
    """First-level block constants of a double-quantised 4-bit weight.

    For block b:  level = absmax_codebook[absmax_codes[b]];
    m = level * absmax_scale[b // blocksize2] (one IEEE float32 multiply,
    round to nearest even); absmax[b] = m + absmax_offset (one float32
    add, round to nearest even).  Returns float32 [nblocks].
    ([DD] 1.4 double quantisation: the quantisation constants are
    themselves quantised.  The page gives no parameters; the 8-bit codes
    through a 256-level table, one float32 scale per 256 blocks and one
    float32 offset are this implementation's reading.)
    """
    if blocksize2 != 256:
        raise ValueError("unsupported second-level block size")
    c8 = np.asarray(absmax_codes, dtype=np.uint8).reshape(-1)[:nblocks]
    if c8.size != nblocks:
        raise ValueError("too few 8-bit codes")
    table = np.asarray(absmax_codebook, dtype=np.float32).reshape(-1)
    if table.size != 256:
        raise ValueError("the 8-bit table has 256 levels")
    sc = np.asarray(absmax_scale, dtype=np.float32).reshape(-1)
    group = np.arange(nblocks) // blocksize2
    if sc.size <= int(group.max(initial=-1)):
        raise ValueError("too few second-level scales")
    m = table[c8] * sc[group]                         # float32 * float32 -> float32
    return (m + np.float32(absmax_offset)).astype(np.float32)   # float32 + float32


def decode_q4dq_bits(codes, absmax_codes, absmax_codebook, absmax_scale, absmax_offset,
                     codebook, n, k, blocksize=64, blocksize2=256) -> np.ndarray:
    """Decode a 4-bit weight whose block constants are double-quantised:
    the constants first (decode_absmax_dq), then the plain 4-bit decode."""
    if blocksize != 64 or (n * k) % blocksize:
        raise ValueError("unsupported 4-bit layout")
    am = decode_absmax_dq(absmax_codes, absmax_codebook, absmax_scale, absmax_offset,
                          (n * k) // blocksize, blocksize2)
    return decode_q4_bits(codes, am, codebook, n, k, blocksize)


def decode_q4_weight(q) -> np.ndarray:
    """Float64 values of a 4-bit weight container with fields codes,
    codebook, n, k and either absmax or the double-quantised constants."""
    if getattr(q, "absmax_codes", None) is not None:
        bits = decode_q4dq_bits(q.codes, q.absmax_codes, q.absmax_codebook, q.absmax_scale,
                                q.absmax_offset, q.codebook, q.n, q.k, q.blocksize,
                                q.absmax_blocksize)
        return bf16_bits_to_f64(bits)
    return decode_q4(q.codes, q.absmax, q.codebook, q.n, q.k, q.blocksize)


# ---------------------------------------------------------------------------
# RMSNorm (the step in front of the gate/up and q/k/v projections)
# ---------------------------------------------------------------------------
def rmsnorm_fwd(X, w, eps):
    """Y = X * rstd * w with rstd = 1 / sqrt(mean_j X[t,j]^2 + eps) per row.

    Returns (Y, rstd).  ([TB] 3.2, the RMSNorm kernel: mean of squares of
    the row, reciprocal square root, kept for the backward, then the
    normalised row times the weight; no bias in the Llama-style layer.)
    """
    X, w = _f64(X), _f64(w)
    rstd = 1.0 / np.sqrt(np.mean(X * X, axis=1) + float(eps))
    return X * rstd[:, None] * w[None, :], rstd


def rmsnorm_bwd(X, w, eps, dY):
    """dL/dX of rmsnorm_fwd for upstream dY, derived by hand ([DD] 2.4 style):
    with g = dY * w and r = rstd,  dX_i = r g_i - r^3 X_i (sum_j g_j X_j) / d
    (the weight is frozen, so there is no dw)."""
    X, w, dY = _f64(X), _f64(w), _f64(dY)
    d = X.shape[1]
    r = 1.0 / np.sqrt(np.mean(X * X, axis=1) + float(eps))
    g = dY * w[None, :]
    dot = np.sum(g * X, axis=1)
    return r[:, None] * g - (r ** 3 * dot / d)[:, None] * X


# ---------------------------------------------------------------------------
# comparison
# ---------------------------------------------------------------------------
def rel_fro(x, ref) -> float:
    """||x - ref||_F / ||ref||_F in float64 (0 when both are zero)."""
    x, ref = _f64(x), _f64(ref)
    num = np.linalg.norm((x - ref).ravel())
    den = np.linalg.norm(ref.ravel())
    if den == 0.0:
        return 0.0 if num == 0.0 else float("inf")
    return float(num / den)
