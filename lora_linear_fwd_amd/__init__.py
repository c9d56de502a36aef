"""Python binding of liblora (ctypes; argument marshalling only).

Every step of the LoRA path runs in liblora's HIP kernels.  PyTorch provides
device memory and the current stream.  Importing this module does not touch
the GPU; loading the library fails loudly when it has not been built.

Entry points mirror the C ABI in include/liblora.h:
  lora_linear_fwd, lora_linear_bwd, lora_swiglu_mlp_fwd, lora_swiglu_mlp_bwd,
  lora_dequant4, lora_decode_weight, lora_merge, lora_qkv_fwd, lora_qkv_bwd,
  lora_rmsnorm_fwd, lora_rmsnorm_bwd,
  lora_workspace_bytes, lora_qkv_workspace_bytes, lora_strerror,
  lora_abi_version.
"""
from __future__ import annotations

import ctypes
import os
from dataclasses import dataclass
from typing import Dict, Optional, Union

HERE = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(HERE, "liblora.so")

LORA_F32, LORA_BF16 = 0, 1
LORA_W_DENSE, LORA_W_Q4, LORA_W_Q4_DQ = 0, 1, 2
LORA_FLAG_ACCUMULATE_DX = 1
OP_LINEAR_FWD, OP_LINEAR_BWD, OP_MLP_FWD, OP_MLP_BWD, OP_QKV_FWD, OP_QKV_BWD = 0, 1, 2, 3, 4, 5
LORA_WS_MINIMAL = 0x100
STATUS = {0: "LORA_OK", 1: "LORA_ERR_NULL_POINTER", 2: "LORA_ERR_BAD_SHAPE",
          3: "LORA_ERR_UNSUPPORTED", 4: "LORA_ERR_WORKSPACE", 5: "LORA_ERR_MISALIGNED",
          6: "LORA_ERR_HIP"}

EXPORTS = ["lora_linear_fwd", "lora_linear_bwd", "lora_swiglu_mlp_fwd", "lora_swiglu_mlp_bwd",
           "lora_dequant4", "lora_workspace_bytes", "lora_strerror", "lora_abi_version",
           "lora_debug_time_next", "lora_merge", "lora_qkv_fwd", "lora_qkv_bwd",
           "lora_qkv_workspace_bytes", "lora_decode_weight", "lora_rmsnorm_fwd",
           "lora_rmsnorm_bwd"]
(KC_GATEUP_FWD, KC_DOWN_FWD, KC_DOWN_BWD, KC_GATEUP_BWD, KC_LINEAR_FWD, KC_LINEAR_DX,
 KC_QKV_FWD, KC_QKV_DX) = range(8)


class LoraError(RuntimeError):
    def __init__(self, status: int, where: str):
        self.status = status
        super().__init__(f"{where}: {STATUS.get(status, status)} ({strerror(status)})")


class LoraWeightC(ctypes.Structure):
    _fields_ = [("fmt", ctypes.c_int32), ("blocksize", ctypes.c_int32),
                ("w", ctypes.c_void_p), ("codes", ctypes.c_void_p),
                ("absmax", ctypes.c_void_p), ("codebook", ctypes.c_void_p),
                ("absmax_codes", ctypes.c_void_p), ("absmax_codebook", ctypes.c_void_p),
                ("absmax_scale", ctypes.c_void_p), ("absmax_offset", ctypes.c_float),
                ("absmax_blocksize", ctypes.c_int32)]


_lib = None


def lib():
    """Load liblora.so (built by __graft_entry__.build() or build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        raise RuntimeError(f"liblora is not built ({LIB_PATH} missing); "
                           "run python lora_linear_fwd_amd/build.py")
    L = ctypes.CDLL(LIB_PATH)
    vp, i64, f32, i32, u32, sz = (ctypes.c_void_p, ctypes.c_int64, ctypes.c_float,
                                  ctypes.c_int, ctypes.c_uint32, ctypes.c_size_t)
    W = ctypes.POINTER(LoraWeightC)
    L.lora_linear_fwd.argtypes = [i32, i64, i64, i64, i64, f32, vp, W, vp, vp, vp, vp, sz, vp]
    L.lora_linear_bwd.argtypes = [i32, i64, i64, i64, i64, f32, vp, W, vp, vp, vp, vp, vp, vp,
                                  u32, vp, sz, vp]
    L.lora_swiglu_mlp_fwd.argtypes = [i32, i64, i64, i64, i64, f32, vp, W, vp, vp, W, vp, vp, W,
                                      vp, vp, vp, vp, vp, vp, sz, vp]
    L.lora_swiglu_mlp_bwd.argtypes = [i32, i64, i64, i64, i64, f32, vp, W, vp, vp, W, vp, vp, W,
                                      vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.lora_dequant4.argtypes = [i64, i64, vp, vp, vp, i32, i32, vp, vp]
    L.lora_merge.argtypes = [i32, i64, i64, i64, f32, i32, W, vp, vp, vp, vp]
    L.lora_decode_weight.argtypes = [i64, i64, W, i32, vp, vp]
    L.lora_rmsnorm_fwd.argtypes = [i32, i64, i64, f32, vp, vp, vp, vp, vp]
    L.lora_rmsnorm_bwd.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, u32, vp]
    L.lora_qkv_fwd.argtypes = [i32, i64, i64, i64, i64, i64, f32, vp, W, vp, vp, W, vp, vp, W, vp,
                               vp, vp, vp, vp, vp, sz, vp]
    L.lora_qkv_bwd.argtypes = [i32, i64, i64, i64, i64, i64, f32, vp, W, vp, vp, W, vp, vp, W, vp,
                               vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp, sz, vp]
    L.lora_qkv_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i64, i64, i64]
    L.lora_qkv_workspace_bytes.restype = sz
    L.lora_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i64, i64]
    L.lora_workspace_bytes.restype = sz
    L.lora_strerror.argtypes = [i32]
    L.lora_strerror.restype = ctypes.c_char_p
    L.lora_abi_version.argtypes = []
    L.lora_debug_time_next.argtypes = [i32, vp, vp]
    L.lora_debug_time_next.restype = ctypes.c_int
    for name in ("lora_linear_fwd", "lora_linear_bwd", "lora_swiglu_mlp_fwd",
                 "lora_swiglu_mlp_bwd", "lora_dequant4", "lora_abi_version", "lora_merge",
                 "lora_qkv_fwd", "lora_qkv_bwd", "lora_decode_weight", "lora_rmsnorm_fwd",
                 "lora_rmsnorm_bwd"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().lora_strerror(status).decode()


def abi_version() -> int:
    return lib().lora_abi_version()


def time_next(kernel_class: int, start_event, stop_event):
    """Have the next launch of GEMM `kernel_class` record the two
    torch.cuda.Event objects around it on the library's launch stream."""
    for ev in (start_event, stop_event):
        if ev.cuda_event == 0:
            ev.record()          # creates the underlying hipEvent
    _check(lib().lora_debug_time_next(kernel_class, ctypes.c_void_p(start_event.cuda_event),
                                      ctypes.c_void_p(stop_event.cuda_event)),
           "lora_debug_time_next")


def workspace_bytes(op, dtype, wfmt, T, k_or_d, n_or_f, r) -> int:
    return int(lib().lora_workspace_bytes(op, dtype, wfmt, T, k_or_d, n_or_f, r))


# --------------------------------------------------------------- tensors
def _torch():
    import torch
    return torch


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream(stream=None):
    torch = _torch()
    s = stream if stream is not None else torch.cuda.current_stream()
    return ctypes.c_void_p(s.cuda_stream)


def _check(status, where):
    if status != 0:
        raise LoraError(status, where)


def _dtype_code(t):
    torch = _torch()
    if t.dtype == torch.bfloat16:
        return LORA_BF16
    if t.dtype == torch.float32:
        return LORA_F32
    raise TypeError(f"unsupported dtype {t.dtype}")


@dataclass
class Q4Weight:
    """4-bit base weight on the device: codes [n, k/2] uint8, absmax
    [n*k/64] fp32, codebook [16] fp32 (layout of include/liblora.h).

    Double-quantised form (absmax_codes set, absmax None): absmax_codes
    [n*k/64] uint8, absmax_codebook [256] fp32, absmax_scale
    [ceil(n*k/64/256)] fp32 and the float absmax_offset."""
    n: int
    k: int
    codes: object
    absmax: object
    codebook: object
    blocksize: int = 64
    absmax_codes: object = None
    absmax_codebook: object = None
    absmax_scale: object = None
    absmax_offset: float = 0.0
    absmax_blocksize: int = 256

    @property
    def double_quant(self) -> bool:
        return self.absmax_codes is not None

    @property
    def shape(self):
        return (self.n, self.k)


Weight = Union["torch.Tensor", Q4Weight]


def _wstruct(W) -> LoraWeightC:
    if isinstance(W, Q4Weight):
        if W.double_quant:
            return LoraWeightC(LORA_W_Q4_DQ, W.blocksize, None, W.codes.data_ptr(), None,
                               W.codebook.data_ptr(), W.absmax_codes.data_ptr(),
                               W.absmax_codebook.data_ptr(), W.absmax_scale.data_ptr(),
                               float(W.absmax_offset), W.absmax_blocksize)
        return LoraWeightC(LORA_W_Q4, W.blocksize, None, W.codes.data_ptr(),
                           W.absmax.data_ptr(), W.codebook.data_ptr())
    return LoraWeightC(LORA_W_DENSE, 0, W.data_ptr(), None, None, None)


def _wfmt(W):
    if isinstance(W, Q4Weight):
        return LORA_W_Q4_DQ if W.double_quant else LORA_W_Q4
    return LORA_W_DENSE


_ws_cache: Dict[tuple, object] = {}


def _workspace(op, dt, wfmt, dims, device, workspace=None, minimal=False):
    """(pointer, byte count) of the workspace handed to the library: the
    caller's tensor at its full size, else a cached buffer passed at exactly
    the size of the requested strategy (fast, or minimal-memory)."""
    torch = _torch()
    if workspace is not None:
        return _ptr(workspace), workspace.numel() * workspace.element_size()
    flag = LORA_WS_MINIMAL if minimal else 0
    if op in (OP_QKV_FWD, OP_QKV_BWD):
        nbytes = int(lib().lora_qkv_workspace_bytes(op | flag, dt, wfmt, *dims))
    else:
        nbytes = workspace_bytes(op | flag, dt, wfmt, *dims)
    if nbytes == 0:
        return None, 0
    key = (str(device), torch.cuda.current_stream(device).cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        buf = torch.empty(nbytes, dtype=torch.uint8, device=device)
        _ws_cache[key] = buf
    return _ptr(buf), nbytes


def clear_workspace_cache():
    _ws_cache.clear()


# ------------------------------------------------------------ entry points
def lora_linear_fwd(X, W: Weight, A, B, alpha: float, Y=None, workspace=None, stream=None,
                    minimal_workspace=False):
    """Y = X W^T + (alpha/r) (X A^T) B^T."""
    torch = _torch()
    T, k = X.shape
    r = A.shape[0]
    n = W.shape[0]
    dt = _dtype_code(X)
    if Y is None:
        Y = torch.empty((T, n), dtype=X.dtype, device=X.device)
    wsp, wsn = _workspace(OP_LINEAR_FWD, dt, _wfmt(W), (T, k, n, r), X.device, workspace,
                          minimal_workspace)
    wst = _wstruct(W)
    _check(lib().lora_linear_fwd(dt, T, k, n, r, float(alpha), _ptr(X), ctypes.byref(wst),
                                 _ptr(A), _ptr(B), _ptr(Y), wsp, wsn, _stream(stream)),
           "lora_linear_fwd")
    return Y


def lora_linear_bwd(X, W: Weight, A, B, alpha: float, dY, need_dx=True, dX=None,
                    accumulate_dx=False, dA=None, dB=None, workspace=None, stream=None,
                    minimal_workspace=False):
    """Returns (dX or None, dA, dB)."""
    torch = _torch()
    T, k = X.shape
    r = A.shape[0]
    n = W.shape[0]
    dt = _dtype_code(X)
    if need_dx and dX is None:
        dX = torch.empty((T, k), dtype=X.dtype, device=X.device)
    if not need_dx:
        dX = None
    dA = torch.empty_like(A) if dA is None else dA
    dB = torch.empty_like(B) if dB is None else dB
    wsp, wsn = _workspace(OP_LINEAR_BWD, dt, _wfmt(W), (T, k, n, r), X.device, workspace,
                          minimal_workspace)
    wst = _wstruct(W)
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate_dx else 0
    _check(lib().lora_linear_bwd(dt, T, k, n, r, float(alpha), _ptr(X), ctypes.byref(wst),
                                 _ptr(A), _ptr(B), _ptr(dY), _ptr(dX), _ptr(dA), _ptr(dB),
                                 flags, wsp, wsn, _stream(stream)),
           "lora_linear_bwd")
    return dX, dA, dB


def _mlp_dims(X, W, A):
    T, d = X.shape
    f = W["gate"].shape[0]
    r = A["gate"].shape[0]
    return T, d, f, r


def lora_swiglu_mlp_fwd(X, W: Dict[str, Weight], A, B, alpha: float, Y=None, e=None, g=None,
                        workspace=None, stream=None, minimal_workspace=False):
    """Returns (Y, e, g); W/A/B are dicts keyed 'gate', 'up', 'down'."""
    torch = _torch()
    T, d, f, r = _mlp_dims(X, W, A)
    dt = _dtype_code(X)
    Y = torch.empty((T, d), dtype=X.dtype, device=X.device) if Y is None else Y
    e = torch.empty((T, f), dtype=X.dtype, device=X.device) if e is None else e
    g = torch.empty((T, f), dtype=X.dtype, device=X.device) if g is None else g
    wsp, wsn = _workspace(OP_MLP_FWD, dt, _wfmt(W["gate"]), (T, d, f, r), X.device, workspace,
                          minimal_workspace)
    ws_ = [_wstruct(W[p]) for p in ("gate", "up", "down")]
    _check(lib().lora_swiglu_mlp_fwd(
        dt, T, d, f, r, float(alpha), _ptr(X),
        ctypes.byref(ws_[0]), _ptr(A["gate"]), _ptr(B["gate"]),
        ctypes.byref(ws_[1]), _ptr(A["up"]), _ptr(B["up"]),
        ctypes.byref(ws_[2]), _ptr(A["down"]), _ptr(B["down"]),
        _ptr(Y), _ptr(e), _ptr(g), wsp, wsn, _stream(stream)),
        "lora_swiglu_mlp_fwd")
    return Y, e, g


def lora_swiglu_mlp_bwd(X, W: Dict[str, Weight], A, B, alpha: float, e, g, dY, need_dx=True,
                        out: Optional[dict] = None, workspace=None, stream=None,
                        minimal_workspace=False):
    """Returns dict with dX (or None) and dA_*/dB_* per projection."""
    torch = _torch()
    T, d, f, r = _mlp_dims(X, W, A)
    dt = _dtype_code(X)
    o = dict(out or {})
    if need_dx and o.get("dX") is None:
        o["dX"] = torch.empty((T, d), dtype=X.dtype, device=X.device)
    if not need_dx:
        o["dX"] = None
    for p in ("gate", "up", "down"):
        if o.get("dA_" + p) is None:
            o["dA_" + p] = torch.empty_like(A[p])
        if o.get("dB_" + p) is None:
            o["dB_" + p] = torch.empty_like(B[p])
    wsp, wsn = _workspace(OP_MLP_BWD, dt, _wfmt(W["gate"]), (T, d, f, r), X.device, workspace,
                          minimal_workspace)
    ws_ = [_wstruct(W[p]) for p in ("gate", "up", "down")]
    _check(lib().lora_swiglu_mlp_bwd(
        dt, T, d, f, r, float(alpha), _ptr(X),
        ctypes.byref(ws_[0]), _ptr(A["gate"]), _ptr(B["gate"]),
        ctypes.byref(ws_[1]), _ptr(A["up"]), _ptr(B["up"]),
        ctypes.byref(ws_[2]), _ptr(A["down"]), _ptr(B["down"]),
        _ptr(e), _ptr(g), _ptr(dY), _ptr(o["dX"]),
        _ptr(o["dA_gate"]), _ptr(o["dB_gate"]), _ptr(o["dA_up"]), _ptr(o["dB_up"]),
        _ptr(o["dA_down"]), _ptr(o["dB_down"]),
        wsp, wsn, _stream(stream)),
        "lora_swiglu_mlp_bwd")
    return o


def lora_qkv_fwd(X, W: Dict[str, Weight], A, B, alpha: float, out: Optional[dict] = None,
                 workspace=None, stream=None, minimal_workspace=False):
    """Returns dict q, k, v of the three LoRA projections of X; W/A/B are
    dicts keyed 'q', 'k', 'v'."""
    torch = _torch()
    T, k = X.shape
    nq, nkv = W["q"].shape[0], W["k"].shape[0]
    r = A["q"].shape[0]
    dt = _dtype_code(X)
    o = dict(out or {})
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        if o.get(p) is None:
            o[p] = torch.empty((T, n), dtype=X.dtype, device=X.device)
    wsp, wsn = _workspace(OP_QKV_FWD, dt, _wfmt(W["q"]), (T, k, nq, nkv, r), X.device, workspace,
                          minimal_workspace)
    ws_ = [_wstruct(W[p]) for p in ("q", "k", "v")]
    _check(lib().lora_qkv_fwd(
        dt, T, k, nq, nkv, r, float(alpha), _ptr(X),
        ctypes.byref(ws_[0]), _ptr(A["q"]), _ptr(B["q"]),
        ctypes.byref(ws_[1]), _ptr(A["k"]), _ptr(B["k"]),
        ctypes.byref(ws_[2]), _ptr(A["v"]), _ptr(B["v"]),
        _ptr(o["q"]), _ptr(o["k"]), _ptr(o["v"]), wsp, wsn, _stream(stream)), "lora_qkv_fwd")
    return o


def lora_qkv_bwd(X, W: Dict[str, Weight], A, B, alpha: float, dY: Dict[str, object],
                 need_dx=True, dX=None, accumulate_dx=False, out: Optional[dict] = None,
                 workspace=None, stream=None, minimal_workspace=False):
    """Returns dict dX (or None) and dA_p / dB_p for p in q, k, v."""
    torch = _torch()
    T, k = X.shape
    nq, nkv = W["q"].shape[0], W["k"].shape[0]
    r = A["q"].shape[0]
    dt = _dtype_code(X)
    o = dict(out or {})
    if need_dx:
        if dX is not None:
            o["dX"] = dX
        elif o.get("dX") is None:
            o["dX"] = torch.empty((T, k), dtype=X.dtype, device=X.device)
    else:
        o["dX"] = None
    for p in ("q", "k", "v"):
        if o.get("dA_" + p) is None:
            o["dA_" + p] = torch.empty_like(A[p])
        if o.get("dB_" + p) is None:
            o["dB_" + p] = torch.empty_like(B[p])
    wsp, wsn = _workspace(OP_QKV_BWD, dt, _wfmt(W["q"]), (T, k, nq, nkv, r), X.device, workspace,
                          minimal_workspace)
    ws_ = [_wstruct(W[p]) for p in ("q", "k", "v")]
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate_dx else 0
    _check(lib().lora_qkv_bwd(
        dt, T, k, nq, nkv, r, float(alpha), _ptr(X),
        ctypes.byref(ws_[0]), _ptr(A["q"]), _ptr(B["q"]),
        ctypes.byref(ws_[1]), _ptr(A["k"]), _ptr(B["k"]),
        ctypes.byref(ws_[2]), _ptr(A["v"]), _ptr(B["v"]),
        _ptr(dY["q"]), _ptr(dY["k"]), _ptr(dY["v"]), _ptr(o["dX"]),
        _ptr(o["dA_q"]), _ptr(o["dB_q"]), _ptr(o["dA_k"]), _ptr(o["dB_k"]),
        _ptr(o["dA_v"]), _ptr(o["dB_v"]), flags, wsp, wsn, _stream(stream)), "lora_qkv_bwd")
    return o


def lora_merge(W: Weight, A, B, alpha: float, sign: int = 1, out=None, stream=None):
    """W + sign * (alpha/r) B A as a new [n, k] tensor (bf16 for 4-bit W)."""
    torch = _torch()
    r = A.shape[0]
    n, k = (W.n, W.k) if isinstance(W, Q4Weight) else W.shape
    dt = _dtype_code(A)
    if out is None:
        out = torch.empty((n, k), dtype=A.dtype, device=A.device)
    wst = _wstruct(W)
    _check(lib().lora_merge(dt, n, k, r, float(alpha), int(sign), ctypes.byref(wst), _ptr(A),
                            _ptr(B), _ptr(out), _stream(stream)),
           "lora_merge")
    return out


def lora_dequant4(q: Q4Weight, out=None, stream=None):
    """Decode a 4-bit weight to a bf16 [n, k] tensor."""
    torch = _torch()
    if out is None:
        out = torch.empty((q.n, q.k), dtype=torch.bfloat16, device=q.codes.device)
    _check(lib().lora_dequant4(q.n, q.k, _ptr(q.codes), _ptr(q.absmax), _ptr(q.codebook),
                               q.blocksize, LORA_BF16, _ptr(out), _stream(stream)),
           "lora_dequant4")
    return out


def lora_rmsnorm_fwd(X, w, eps: float, Y=None, rstd=None, stream=None):
    """RMSNorm of the rows of X: returns (Y, rstd) with rstd [T] fp32."""
    torch = _torch()
    T, d = X.shape
    dt = _dtype_code(X)
    if Y is None:
        Y = torch.empty_like(X)
    if rstd is None:
        rstd = torch.empty((T,), dtype=torch.float32, device=X.device)
    _check(lib().lora_rmsnorm_fwd(dt, T, d, float(eps), _ptr(X), _ptr(w), _ptr(Y), _ptr(rstd),
                                  _stream(stream)), "lora_rmsnorm_fwd")
    return Y, rstd


def lora_rmsnorm_bwd(X, w, rstd, dY, dX=None, accumulate=False, stream=None):
    """Input gradient of lora_rmsnorm_fwd (added to dX when accumulate)."""
    torch = _torch()
    T, d = X.shape
    dt = _dtype_code(X)
    if dX is None:
        if accumulate:
            raise ValueError("accumulate needs dX")
        dX = torch.empty_like(X)
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate else 0
    _check(lib().lora_rmsnorm_bwd(dt, T, d, _ptr(X), _ptr(w), _ptr(rstd), _ptr(dY), _ptr(dX),
                                  flags, _stream(stream)), "lora_rmsnorm_bwd")
    return dX


def lora_decode_weight(q: Q4Weight, out=None, stream=None):
    """Decode a 4-bit weight of either form (plain or double-quantised
    block constants) to a bf16 [n, k] tensor."""
    torch = _torch()
    if out is None:
        out = torch.empty((q.n, q.k), dtype=torch.bfloat16, device=q.codes.device)
    wst = _wstruct(q)
    _check(lib().lora_decode_weight(q.n, q.k, ctypes.byref(wst), LORA_BF16, _ptr(out),
                                    _stream(stream)), "lora_decode_weight")
    return out


# ------------------------------------------------------ host -> device helpers
def to_device_q4(qw, device="cuda"):
    """Upload a host-side lora_inputs.Q4Weight (either form)."""
    torch = _torch()

    def up(a):
        return None if a is None else torch.from_numpy(a).to(device)
    return Q4Weight(qw.n, qw.k, up(qw.codes), up(qw.absmax), up(qw.codebook), qw.blocksize,
                    up(qw.absmax_codes), up(qw.absmax_codebook), up(qw.absmax_scale),
                    float(qw.absmax_offset), qw.absmax_blocksize)
