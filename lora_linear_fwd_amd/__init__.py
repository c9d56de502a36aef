"""Python binding of liblora (ctypes; argument marshalling only).

Every step of the LoRA path runs in liblora's HIP kernels.  PyTorch provides
device memory and the current stream.  Importing this module does not touch
the GPU; loading the library fails loudly when it has not been built.  Every
tensor argument is checked (shape against the derived sizes, dtype, device,
contiguity) before the library is called: the C ABI takes bare pointers and
assumes row-major contiguous tensors of the stated shapes.

Entry points mirror the C ABI in include/liblora.h:
  lora_linear_fwd, lora_linear_bwd, lora_swiglu_mlp_fwd, lora_swiglu_mlp_bwd,
  lora_dequant4, lora_decode_weight, lora_merge, lora_qkv_fwd, lora_qkv_bwd,
  lora_rmsnorm_fwd, lora_rmsnorm_bwd, lora_linear_bwd_noalloc,
  lora_rmsnorm_swiglu_mlp_fwd, lora_rmsnorm_swiglu_mlp_bwd, lora_fold_norm_weight,
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
# the same kernels with the GEMM timing hook of include/liblora_timing.h
TIMED_LIB_PATH = os.path.join(HERE, "liblora_timed.so")

LORA_F32, LORA_BF16 = 0, 1
LORA_W_DENSE, LORA_W_Q4, LORA_W_Q4_DQ = 0, 1, 2
LORA_FLAG_ACCUMULATE_DX = 1
OP_LINEAR_FWD, OP_LINEAR_BWD, OP_MLP_FWD, OP_MLP_BWD, OP_QKV_FWD, OP_QKV_BWD = 0, 1, 2, 3, 4, 5
OP_RMSNORM_MLP_FWD, OP_RMSNORM_MLP_BWD = 6, 7
OP_RMSNORM_QKV_FWD, OP_RMSNORM_QKV_BWD = 8, 9
LORA_WS_MINIMAL = 0x100
STATUS = {0: "LORA_OK", 1: "LORA_ERR_NULL_POINTER", 2: "LORA_ERR_BAD_SHAPE",
          3: "LORA_ERR_UNSUPPORTED", 4: "LORA_ERR_WORKSPACE", 5: "LORA_ERR_MISALIGNED",
          6: "LORA_ERR_HIP"}

EXPORTS = ["lora_linear_fwd", "lora_linear_bwd", "lora_swiglu_mlp_fwd", "lora_swiglu_mlp_bwd",
           "lora_dequant4", "lora_workspace_bytes", "lora_strerror", "lora_abi_version",
           "lora_merge", "lora_qkv_fwd", "lora_qkv_bwd",
           "lora_qkv_workspace_bytes", "lora_decode_weight", "lora_rmsnorm_fwd",
           "lora_rmsnorm_bwd", "lora_linear_bwd_noalloc", "lora_rmsnorm_swiglu_mlp_fwd",
           "lora_rmsnorm_swiglu_mlp_bwd", "lora_fold_norm_weight", "lora_rmsnorm_qkv_fwd",
           "lora_rmsnorm_qkv_bwd"]
TIMING_EXPORTS = ["lora_debug_time_next"]
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
                ("absmax_blocksize", ctypes.c_int32), ("wt", ctypes.c_void_p)]


_lib = None
_lib_path = LIB_PATH


def use_timing_build():
    """Load liblora_timed.so instead of liblora.so (same kernels, plus the
    GEMM timing hook).  Must be called before the first library call."""
    global _lib_path
    if _lib is not None and _lib_path != TIMED_LIB_PATH:
        raise RuntimeError("liblora.so is already loaded")
    _lib_path = TIMED_LIB_PATH


def lib():
    """Load liblora.so (built by __graft_entry__.build() or build.py)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(_lib_path):
        raise RuntimeError(f"liblora is not built ({_lib_path} missing); "
                           "run python lora_linear_fwd_amd/build.py")
    L = ctypes.CDLL(_lib_path)
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
    L.lora_linear_bwd_noalloc.argtypes = [i32, i64, i64, i64, i64, f32, vp, W, vp, vp, vp, vp,
                                          vp, vp, u32, vp]
    L.lora_dequant4.argtypes = [i64, i64, vp, vp, vp, i32, i32, vp, vp]
    L.lora_rmsnorm_swiglu_mlp_fwd.argtypes = [i32, i64, i64, i64, i64, f32, f32, vp, vp, W, vp, vp,
                                              W, vp, vp, W, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.lora_rmsnorm_swiglu_mlp_bwd.argtypes = [i32, i64, i64, i64, i64, f32, vp, vp, vp, W, vp, vp,
                                              W, vp, vp, W, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                              vp, vp, vp, u32, vp, sz, vp]
    L.lora_fold_norm_weight.argtypes = [i32, i64, i64, vp, vp, vp, vp]
    L.lora_merge.argtypes = [i32, i64, i64, i64, f32, i32, W, vp, vp, vp, vp]
    L.lora_decode_weight.argtypes = [i64, i64, W, i32, vp, vp]
    L.lora_rmsnorm_fwd.argtypes = [i32, i64, i64, f32, vp, vp, vp, vp, vp]
    L.lora_rmsnorm_bwd.argtypes = [i32, i64, i64, vp, vp, vp, vp, vp, u32, vp]
    L.lora_qkv_fwd.argtypes = [i32, i64, i64, i64, i64, i64, f32, vp, W, vp, vp, W, vp, vp, W, vp,
                               vp, vp, vp, vp, vp, sz, vp]
    L.lora_qkv_bwd.argtypes = [i32, i64, i64, i64, i64, i64, f32, vp, W, vp, vp, W, vp, vp, W, vp,
                               vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, u32, vp, sz, vp]
    L.lora_rmsnorm_qkv_fwd.argtypes = [i32, i64, i64, i64, i64, i64, f32, f32, vp, vp, W, vp, vp,
                                       W, vp, vp, W, vp, vp, vp, vp, vp, vp, vp, sz, vp]
    L.lora_rmsnorm_qkv_bwd.argtypes = [i32, i64, i64, i64, i64, i64, f32, vp, vp, vp, W, vp, vp,
                                       W, vp, vp, W, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp,
                                       vp, u32, vp, sz, vp]
    L.lora_qkv_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i64, i64, i64]
    L.lora_qkv_workspace_bytes.restype = sz
    L.lora_workspace_bytes.argtypes = [i32, i32, i32, i64, i64, i64, i64]
    L.lora_workspace_bytes.restype = sz
    L.lora_strerror.argtypes = [i32]
    L.lora_strerror.restype = ctypes.c_char_p
    L.lora_abi_version.argtypes = []
    if _lib_path == TIMED_LIB_PATH:
        L.lora_debug_time_next.argtypes = [i32, vp, vp]
        L.lora_debug_time_next.restype = ctypes.c_int
    for name in ("lora_linear_fwd", "lora_linear_bwd", "lora_swiglu_mlp_fwd",
                 "lora_swiglu_mlp_bwd", "lora_dequant4", "lora_abi_version", "lora_merge",
                 "lora_qkv_fwd", "lora_qkv_bwd", "lora_decode_weight", "lora_rmsnorm_fwd",
                 "lora_rmsnorm_bwd", "lora_linear_bwd_noalloc", "lora_rmsnorm_swiglu_mlp_fwd",
                 "lora_rmsnorm_swiglu_mlp_bwd", "lora_fold_norm_weight"):
        getattr(L, name).restype = ctypes.c_int
    _lib = L
    return L


def strerror(status: int) -> str:
    return lib().lora_strerror(status).decode()


def abi_version() -> int:
    return lib().lora_abi_version()


def time_next(kernel_class: int, start_event, stop_event):
    """Have the calling thread's next launch of GEMM `kernel_class` record
    the two torch.cuda.Event objects around it on the library's launch
    stream (timing build only: see use_timing_build)."""
    if _lib_path != TIMED_LIB_PATH:
        raise RuntimeError("time_next needs the timing build (use_timing_build())")
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


def _stream_obj(stream=None):
    torch = _torch()
    return stream if stream is not None else torch.cuda.current_stream()


def _stream(stream=None):
    return ctypes.c_void_p(_stream_obj(stream).cuda_stream)


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


# ------------------------------------------------------- argument checks
def _need(cond, msg):
    if not cond:
        raise ValueError(msg)


def _tensor(t, name, shape, dtype, device, where):
    """t must be a contiguous tensor of exactly `shape` (None entries: any
    size), `dtype` and `device`."""
    torch = _torch()
    _need(isinstance(t, torch.Tensor), f"{where}: {name} must be a tensor")
    _need(t.dim() == len(shape) and all(s is None or int(a) == int(s)
                                        for a, s in zip(t.shape, shape)),
          f"{where}: {name} has shape {tuple(t.shape)}, expected "
          f"{tuple('*' if s is None else int(s) for s in shape)}")
    _need(t.dtype == dtype, f"{where}: {name} has dtype {t.dtype}, expected {dtype}")
    _need(t.device == device, f"{where}: {name} is on {t.device}, expected {device}")
    _need(t.is_contiguous(), f"{where}: {name} must be contiguous (row-major)")


def _on_gpu(X, where):
    _need(X.device.type == "cuda", f"{where}: tensors must be on a GPU (got {X.device})")


def _weight(W, name, n, k, dtype, device, where):
    """A dense [n, k] tensor of the call's dtype, or a Q4Weight of that
    logical shape with every container field in the layout liblora.h
    states."""
    torch = _torch()
    if isinstance(W, Q4Weight):
        _need((W.n, W.k) == (n, k), f"{where}: {name} is {W.n}x{W.k}, expected {n}x{k}")
        _need(dtype == torch.bfloat16, f"{where}: 4-bit weights need bf16 activations")
        _need(W.blocksize == 64 and k % 64 == 0, f"{where}: {name}: blocksize 64, k % 64 == 0")
        nblk = n * k // 64
        _tensor(W.codes.reshape(-1) if W.codes.is_contiguous() else W.codes, name + ".codes",
                (n * k // 2,), torch.uint8, device, where)
        _tensor(W.codebook, name + ".codebook", (16,), torch.float32, device, where)
        if W.double_quant:
            _need(W.absmax_blocksize == 256, f"{where}: {name}: absmax_blocksize 256")
            _tensor(W.absmax_codes.reshape(-1) if W.absmax_codes.is_contiguous()
                    else W.absmax_codes, name + ".absmax_codes", (nblk,), torch.uint8, device,
                    where)
            _tensor(W.absmax_codebook, name + ".absmax_codebook", (256,), torch.float32,
                    device, where)
            _tensor(W.absmax_scale.reshape(-1) if W.absmax_scale.is_contiguous()
                    else W.absmax_scale, name + ".absmax_scale", ((nblk + 255) // 256,),
                    torch.float32, device, where)
        else:
            _tensor(W.absmax.reshape(-1) if W.absmax.is_contiguous() else W.absmax,
                    name + ".absmax", (nblk,), torch.float32, device, where)
    elif isinstance(W, DenseWeight):
        _tensor(W.w, name, (n, k), dtype, device, where)
        _tensor(W.wt, name + ".wt", (k, n), dtype, device, where)
    else:
        _tensor(W, name, (n, k), dtype, device, where)


def _adapter(A, B, n, k, r, dtype, device, where, suffix=""):
    _tensor(A, "A" + suffix, (r, k), dtype, device, where)
    _tensor(B, "B" + suffix, (n, r), dtype, device, where)


def _x(X, where):
    torch = _torch()
    _need(isinstance(X, torch.Tensor) and X.dim() == 2, f"{where}: X must be a 2-D tensor")
    _dtype_code(X)
    _need(X.is_contiguous(), f"{where}: X must be contiguous (row-major)")
    return X.shape[0], X.shape[1]


def _rank(A, where):
    torch = _torch()
    _need(isinstance(A, torch.Tensor) and A.dim() == 2, f"{where}: A must be a 2-D tensor")
    return A.shape[0]


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


@dataclass
class DenseWeight:
    """A dense frozen base weight w [n, k] with a copy of its transpose wt
    [k, n] kept next to it (made once): the backward dX products then run the
    K-contiguous GEMM form on wt.  Build with with_transpose(w)."""
    w: object
    wt: object

    @property
    def shape(self):
        return tuple(self.w.shape)


def with_transpose(w):
    """DenseWeight(w, w^T as a contiguous copy)."""
    return DenseWeight(w, w.t().contiguous())


Weight = Union["torch.Tensor", Q4Weight, DenseWeight]


def _wstruct(W) -> LoraWeightC:
    if isinstance(W, Q4Weight):
        if W.double_quant:
            return LoraWeightC(LORA_W_Q4_DQ, W.blocksize, None, W.codes.data_ptr(), None,
                               W.codebook.data_ptr(), W.absmax_codes.data_ptr(),
                               W.absmax_codebook.data_ptr(), W.absmax_scale.data_ptr(),
                               float(W.absmax_offset), W.absmax_blocksize)
        return LoraWeightC(LORA_W_Q4, W.blocksize, None, W.codes.data_ptr(),
                           W.absmax.data_ptr(), W.codebook.data_ptr())
    if isinstance(W, DenseWeight):
        return LoraWeightC(LORA_W_DENSE, 0, W.w.data_ptr(), None, None, None, None, None, None,
                           0.0, 0, W.wt.data_ptr())
    return LoraWeightC(LORA_W_DENSE, 0, W.data_ptr(), None, None, None)


def _wfmt(W):
    if isinstance(W, Q4Weight):
        return LORA_W_Q4_DQ if W.double_quant else LORA_W_Q4
    return LORA_W_DENSE


_ws_cache: Dict[tuple, object] = {}


def _workspace(op, dt, wfmt, dims, device, workspace=None, minimal=False, stream=None):
    """(pointer, byte count) of the workspace handed to the library: the
    caller's tensor at its full size, else a buffer cached per device and
    per the stream the kernels run on, passed at exactly the size of the
    requested strategy (fast, or minimal-memory).  A cached buffer is
    allocated on that stream, so the caching allocator does not hand its
    memory to other streams' work while this stream may still use it."""
    torch = _torch()
    if workspace is not None:
        _need(workspace.device == device and workspace.is_contiguous(),
              "workspace must be a contiguous tensor on the inputs' device")
        return _ptr(workspace), workspace.numel() * workspace.element_size()
    flag = LORA_WS_MINIMAL if minimal else 0
    if op in (OP_QKV_FWD, OP_QKV_BWD, OP_RMSNORM_QKV_FWD, OP_RMSNORM_QKV_BWD):
        nbytes = int(lib().lora_qkv_workspace_bytes(op | flag, dt, wfmt, *dims))
    else:
        nbytes = workspace_bytes(op | flag, dt, wfmt, *dims)
    if nbytes == 0:
        return None, 0
    s = _stream_obj(stream)
    key = (str(device), s.cuda_stream)
    buf = _ws_cache.get(key)
    if buf is None or buf.numel() < nbytes:
        with torch.cuda.stream(s):
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
    where = "lora_linear_fwd"
    T, k = _x(X, where)
    r = _rank(A, where)
    n = W.shape[0]
    _weight(W, "W", n, k, X.dtype, X.device, where)
    _adapter(A, B, n, k, r, X.dtype, X.device, where)
    if Y is not None:
        _tensor(Y, "Y", (T, n), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    if Y is None:
        Y = torch.empty((T, n), dtype=X.dtype, device=X.device)
    wsp, wsn = _workspace(OP_LINEAR_FWD, dt, _wfmt(W), (T, k, n, r), X.device, workspace,
                          minimal_workspace, stream)
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
    where = "lora_linear_bwd"
    T, k = _x(X, where)
    r = _rank(A, where)
    n = W.shape[0]
    _weight(W, "W", n, k, X.dtype, X.device, where)
    _adapter(A, B, n, k, r, X.dtype, X.device, where)
    _tensor(dY, "dY", (T, n), X.dtype, X.device, where)
    _need(not accumulate_dx or (need_dx and dX is not None), f"{where}: accumulate_dx needs dX")
    if need_dx and dX is not None:
        _tensor(dX, "dX", (T, k), X.dtype, X.device, where)
    if dA is not None:
        _tensor(dA, "dA", (r, k), X.dtype, X.device, where)
    if dB is not None:
        _tensor(dB, "dB", (n, r), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    if need_dx and dX is None:
        dX = torch.empty((T, k), dtype=X.dtype, device=X.device)
    if not need_dx:
        dX = None
    dA = torch.empty_like(A) if dA is None else dA
    dB = torch.empty_like(B) if dB is None else dB
    wsp, wsn = _workspace(OP_LINEAR_BWD, dt, _wfmt(W), (T, k, n, r), X.device, workspace,
                          minimal_workspace, stream)
    wst = _wstruct(W)
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate_dx else 0
    _check(lib().lora_linear_bwd(dt, T, k, n, r, float(alpha), _ptr(X), ctypes.byref(wst),
                                 _ptr(A), _ptr(B), _ptr(dY), _ptr(dX), _ptr(dA), _ptr(dB),
                                 flags, wsp, wsn, _stream(stream)),
           "lora_linear_bwd")
    return dX, dA, dB


LORA_NOALLOC_SCRATCH_BYTES = 128 << 20


def lora_linear_bwd_noalloc(X, W: Weight, A, B, alpha: float, dY, dX, dA, dB,
                            accumulate_dx=False, stream=None):
    """lora_linear_bwd without a workspace: the library's static per-GPU
    scratch array (LORA_NOALLOC_SCRATCH_BYTES) holds its scratch memory.  The
    caller passes every output (dX may be None); nothing is allocated."""
    where = "lora_linear_bwd_noalloc"
    T, k = _x(X, where)
    r = _rank(A, where)
    n = W.shape[0]
    _weight(W, "W", n, k, X.dtype, X.device, where)
    _adapter(A, B, n, k, r, X.dtype, X.device, where)
    _tensor(dY, "dY", (T, n), X.dtype, X.device, where)
    _need(not accumulate_dx or dX is not None, f"{where}: accumulate_dx needs dX")
    if dX is not None:
        _tensor(dX, "dX", (T, k), X.dtype, X.device, where)
    _tensor(dA, "dA", (r, k), X.dtype, X.device, where)
    _tensor(dB, "dB", (n, r), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    wst = _wstruct(W)
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate_dx else 0
    _check(lib().lora_linear_bwd_noalloc(dt, T, k, n, r, float(alpha), _ptr(X),
                                         ctypes.byref(wst), _ptr(A), _ptr(B), _ptr(dY),
                                         _ptr(dX), _ptr(dA), _ptr(dB), flags, _stream(stream)),
           where)
    return dX, dA, dB


_MLP_SHAPES = {"gate": lambda d, f: (f, d), "up": lambda d, f: (f, d), "down": lambda d, f: (d, f)}


def _mlp_check(X, W, A, B, where):
    """(T, d, f, r) of an MLP call, every weight and adapter checked."""
    T, d = _x(X, where)
    _need(all(p in W and p in A and p in B for p in _MLP_SHAPES),
          f"{where}: W, A and B need the keys gate, up, down")
    f = W["gate"].shape[0]
    r = _rank(A["gate"], where)
    for p, shp in _MLP_SHAPES.items():
        n, k = shp(d, f)
        _weight(W[p], "W_" + p, n, k, X.dtype, X.device, where)
        _adapter(A[p], B[p], n, k, r, X.dtype, X.device, where, "_" + p)
    _need(_wfmt(W["gate"]) == _wfmt(W["up"]), f"{where}: gate and up weights share one format")
    return T, d, f, r


def lora_swiglu_mlp_fwd(X, W: Dict[str, Weight], A, B, alpha: float, Y=None, e=None, g=None,
                        workspace=None, stream=None, minimal_workspace=False):
    """Returns (Y, e, g); W/A/B are dicts keyed 'gate', 'up', 'down'."""
    torch = _torch()
    where = "lora_swiglu_mlp_fwd"
    T, d, f, r = _mlp_check(X, W, A, B, where)
    for t, name, shp in ((Y, "Y", (T, d)), (e, "e", (T, f)), (g, "g", (T, f))):
        if t is not None:
            _tensor(t, name, shp, X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    Y = torch.empty((T, d), dtype=X.dtype, device=X.device) if Y is None else Y
    e = torch.empty((T, f), dtype=X.dtype, device=X.device) if e is None else e
    g = torch.empty((T, f), dtype=X.dtype, device=X.device) if g is None else g
    wsp, wsn = _workspace(OP_MLP_FWD, dt, _wfmt(W["gate"]), (T, d, f, r), X.device, workspace,
                          minimal_workspace, stream)
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
    where = "lora_swiglu_mlp_bwd"
    T, d, f, r = _mlp_check(X, W, A, B, where)
    _tensor(e, "e", (T, f), X.dtype, X.device, where)
    _tensor(g, "g", (T, f), X.dtype, X.device, where)
    _tensor(dY, "dY", (T, d), X.dtype, X.device, where)
    o = dict(out or {})
    if need_dx and o.get("dX") is not None:
        _tensor(o["dX"], "dX", (T, d), X.dtype, X.device, where)
    for p, shp in _MLP_SHAPES.items():
        n, k = shp(d, f)
        if o.get("dA_" + p) is not None:
            _tensor(o["dA_" + p], "dA_" + p, (r, k), X.dtype, X.device, where)
        if o.get("dB_" + p) is not None:
            _tensor(o["dB_" + p], "dB_" + p, (n, r), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
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
                          minimal_workspace, stream)
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


def lora_fold_norm_weight(W, w, out=None, stream=None):
    """W diag(w) for a frozen base weight W [n, k] that reads the output of an
    RMSNorm with frozen weight w [k] (bf16; out may be W itself)."""
    torch = _torch()
    where = "lora_fold_norm_weight"
    _need(isinstance(W, torch.Tensor) and W.dim() == 2, f"{where}: W must be a 2-D tensor")
    n, k = W.shape
    _tensor(W, "W", (n, k), torch.bfloat16, W.device, where)
    _tensor(w, "w", (k,), torch.bfloat16, W.device, where)
    if out is not None:
        _tensor(out, "out", (n, k), torch.bfloat16, W.device, where)
    _on_gpu(W, where)
    if out is None:
        out = torch.empty_like(W)
    _check(lib().lora_fold_norm_weight(LORA_BF16, n, k, _ptr(W), _ptr(w), _ptr(out),
                                       _stream(stream)), where)
    return out


def lora_rmsnorm_swiglu_mlp_fwd(X, norm_w, eps: float, W: Dict[str, Weight], A, B, alpha: float,
                                Y=None, e=None, g=None, rstd=None, workspace=None, stream=None):
    """RMSNorm of the raw rows X fused into the LoRA-SwiGLU MLP.  W["gate"]
    and W["up"] must be folded with the norm weight (lora_fold_norm_weight).
    Returns (Y, e, g, rstd)."""
    torch = _torch()
    where = "lora_rmsnorm_swiglu_mlp_fwd"
    T, d, f, r = _mlp_check(X, W, A, B, where)
    _tensor(norm_w, "norm_w", (d,), X.dtype, X.device, where)
    for t, name, shp, dt_ in ((Y, "Y", (T, d), X.dtype), (e, "e", (T, f), X.dtype),
                              (g, "g", (T, f), X.dtype), (rstd, "rstd", (T,), torch.float32)):
        if t is not None:
            _tensor(t, name, shp, dt_, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    Y = torch.empty((T, d), dtype=X.dtype, device=X.device) if Y is None else Y
    e = torch.empty((T, f), dtype=X.dtype, device=X.device) if e is None else e
    g = torch.empty((T, f), dtype=X.dtype, device=X.device) if g is None else g
    rstd = torch.empty((T,), dtype=torch.float32, device=X.device) if rstd is None else rstd
    wsp, wsn = _workspace(OP_RMSNORM_MLP_FWD, dt, _wfmt(W["gate"]), (T, d, f, r), X.device,
                          workspace, False, stream)
    ws_ = [_wstruct(W[p]) for p in ("gate", "up", "down")]
    _check(lib().lora_rmsnorm_swiglu_mlp_fwd(
        dt, T, d, f, r, float(alpha), float(eps), _ptr(X), _ptr(norm_w),
        ctypes.byref(ws_[0]), _ptr(A["gate"]), _ptr(B["gate"]),
        ctypes.byref(ws_[1]), _ptr(A["up"]), _ptr(B["up"]),
        ctypes.byref(ws_[2]), _ptr(A["down"]), _ptr(B["down"]),
        _ptr(Y), _ptr(e), _ptr(g), _ptr(rstd), wsp, wsn, _stream(stream)), where)
    return Y, e, g, rstd


def lora_rmsnorm_swiglu_mlp_bwd(X, norm_w, rstd, W: Dict[str, Weight], A, B, alpha: float, e, g,
                                dY, need_dx=True, accumulate_dx=False, out: Optional[dict] = None,
                                workspace=None, stream=None):
    """Backward of lora_rmsnorm_swiglu_mlp_fwd: dict with dX (gradient of
    the raw rows; added to out["dX"] when accumulate_dx) and dA_*/dB_*."""
    torch = _torch()
    where = "lora_rmsnorm_swiglu_mlp_bwd"
    T, d, f, r = _mlp_check(X, W, A, B, where)
    _tensor(norm_w, "norm_w", (d,), X.dtype, X.device, where)
    _tensor(rstd, "rstd", (T,), torch.float32, X.device, where)
    _tensor(e, "e", (T, f), X.dtype, X.device, where)
    _tensor(g, "g", (T, f), X.dtype, X.device, where)
    _tensor(dY, "dY", (T, d), X.dtype, X.device, where)
    o = dict(out or {})
    if need_dx and o.get("dX") is not None:
        _tensor(o["dX"], "dX", (T, d), X.dtype, X.device, where)
    _need(not accumulate_dx or (need_dx and o.get("dX") is not None),
          f"{where}: accumulate_dx needs out['dX']")
    for p, shp in _MLP_SHAPES.items():
        n, k = shp(d, f)
        if o.get("dA_" + p) is not None:
            _tensor(o["dA_" + p], "dA_" + p, (r, k), X.dtype, X.device, where)
        if o.get("dB_" + p) is not None:
            _tensor(o["dB_" + p], "dB_" + p, (n, r), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    if need_dx and o.get("dX") is None:
        o["dX"] = torch.empty((T, d), dtype=X.dtype, device=X.device)
    if not need_dx:
        o["dX"] = None
    for p in ("gate", "up", "down"):
        if o.get("dA_" + p) is None:
            o["dA_" + p] = torch.empty_like(A[p])
        if o.get("dB_" + p) is None:
            o["dB_" + p] = torch.empty_like(B[p])
    wsp, wsn = _workspace(OP_RMSNORM_MLP_BWD, dt, _wfmt(W["gate"]), (T, d, f, r), X.device,
                          workspace, False, stream)
    ws_ = [_wstruct(W[p]) for p in ("gate", "up", "down")]
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate_dx else 0
    _check(lib().lora_rmsnorm_swiglu_mlp_bwd(
        dt, T, d, f, r, float(alpha), _ptr(X), _ptr(norm_w), _ptr(rstd),
        ctypes.byref(ws_[0]), _ptr(A["gate"]), _ptr(B["gate"]),
        ctypes.byref(ws_[1]), _ptr(A["up"]), _ptr(B["up"]),
        ctypes.byref(ws_[2]), _ptr(A["down"]), _ptr(B["down"]),
        _ptr(e), _ptr(g), _ptr(dY), _ptr(o["dX"]),
        _ptr(o["dA_gate"]), _ptr(o["dB_gate"]), _ptr(o["dA_up"]), _ptr(o["dB_up"]),
        _ptr(o["dA_down"]), _ptr(o["dB_down"]), flags, wsp, wsn, _stream(stream)), where)
    return o


def _qkv_check(X, W, A, B, where):
    T, k = _x(X, where)
    _need(all(p in W and p in A and p in B for p in "qkv"),
          f"{where}: W, A and B need the keys q, k, v")
    nq, nkv = W["q"].shape[0], W["k"].shape[0]
    r = _rank(A["q"], where)
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        _weight(W[p], "W_" + p, n, k, X.dtype, X.device, where)
        _adapter(A[p], B[p], n, k, r, X.dtype, X.device, where, "_" + p)
    _need(_wfmt(W["q"]) == _wfmt(W["k"]) == _wfmt(W["v"]),
          f"{where}: q, k and v weights share one format")
    return T, k, nq, nkv, r


def lora_qkv_fwd(X, W: Dict[str, Weight], A, B, alpha: float, out: Optional[dict] = None,
                 workspace=None, stream=None, minimal_workspace=False):
    """Returns dict q, k, v of the three LoRA projections of X; W/A/B are
    dicts keyed 'q', 'k', 'v'."""
    torch = _torch()
    where = "lora_qkv_fwd"
    T, k, nq, nkv, r = _qkv_check(X, W, A, B, where)
    o = dict(out or {})
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        if o.get(p) is not None:
            _tensor(o[p], p, (T, n), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        if o.get(p) is None:
            o[p] = torch.empty((T, n), dtype=X.dtype, device=X.device)
    wsp, wsn = _workspace(OP_QKV_FWD, dt, _wfmt(W["q"]), (T, k, nq, nkv, r), X.device, workspace,
                          minimal_workspace, stream)
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
    where = "lora_qkv_bwd"
    T, k, nq, nkv, r = _qkv_check(X, W, A, B, where)
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        _tensor(dY[p], "d" + p.upper(), (T, n), X.dtype, X.device, where)
    o = dict(out or {})
    if need_dx:
        if dX is not None:
            o["dX"] = dX
        if o.get("dX") is not None:
            _tensor(o["dX"], "dX", (T, k), X.dtype, X.device, where)
    _need(not accumulate_dx or (need_dx and o.get("dX") is not None),
          f"{where}: accumulate_dx needs dX")
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        if o.get("dA_" + p) is not None:
            _tensor(o["dA_" + p], "dA_" + p, (r, k), X.dtype, X.device, where)
        if o.get("dB_" + p) is not None:
            _tensor(o["dB_" + p], "dB_" + p, (n, r), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    if need_dx:
        if o.get("dX") is None:
            o["dX"] = torch.empty((T, k), dtype=X.dtype, device=X.device)
    else:
        o["dX"] = None
    for p in ("q", "k", "v"):
        if o.get("dA_" + p) is None:
            o["dA_" + p] = torch.empty_like(A[p])
        if o.get("dB_" + p) is None:
            o["dB_" + p] = torch.empty_like(B[p])
    wsp, wsn = _workspace(OP_QKV_BWD, dt, _wfmt(W["q"]), (T, k, nq, nkv, r), X.device, workspace,
                          minimal_workspace, stream)
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


def lora_rmsnorm_qkv_fwd(X, norm_w, eps: float, W: Dict[str, Weight], A, B, alpha: float,
                         out: Optional[dict] = None, rstd=None, workspace=None, stream=None):
    """RMSNorm of the raw rows X fused into the q/k/v LoRA projections.
    W["q"], W["k"], W["v"] must be folded with the norm weight
    (lora_fold_norm_weight).  Returns (dict q, k, v; rstd)."""
    torch = _torch()
    where = "lora_rmsnorm_qkv_fwd"
    T, k, nq, nkv, r = _qkv_check(X, W, A, B, where)
    _tensor(norm_w, "norm_w", (k,), X.dtype, X.device, where)
    o = dict(out or {})
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        if o.get(p) is not None:
            _tensor(o[p], p, (T, n), X.dtype, X.device, where)
    if rstd is not None:
        _tensor(rstd, "rstd", (T,), torch.float32, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        if o.get(p) is None:
            o[p] = torch.empty((T, n), dtype=X.dtype, device=X.device)
    rstd = torch.empty((T,), dtype=torch.float32, device=X.device) if rstd is None else rstd
    wsp, wsn = _workspace(OP_RMSNORM_QKV_FWD, dt, _wfmt(W["q"]), (T, k, nq, nkv, r), X.device,
                          workspace, False, stream)
    ws_ = [_wstruct(W[p]) for p in ("q", "k", "v")]
    _check(lib().lora_rmsnorm_qkv_fwd(
        dt, T, k, nq, nkv, r, float(alpha), float(eps), _ptr(X), _ptr(norm_w),
        ctypes.byref(ws_[0]), _ptr(A["q"]), _ptr(B["q"]),
        ctypes.byref(ws_[1]), _ptr(A["k"]), _ptr(B["k"]),
        ctypes.byref(ws_[2]), _ptr(A["v"]), _ptr(B["v"]),
        _ptr(o["q"]), _ptr(o["k"]), _ptr(o["v"]), _ptr(rstd), wsp, wsn, _stream(stream)), where)
    return o, rstd


def lora_rmsnorm_qkv_bwd(X, norm_w, rstd, W: Dict[str, Weight], A, B, alpha: float,
                         dY: Dict[str, object], need_dx=True, accumulate_dx=False,
                         out: Optional[dict] = None, workspace=None, stream=None):
    """Backward of lora_rmsnorm_qkv_fwd: dict with dX (gradient of the raw
    rows; added to out["dX"] when accumulate_dx) and dA_p / dB_p."""
    torch = _torch()
    where = "lora_rmsnorm_qkv_bwd"
    T, k, nq, nkv, r = _qkv_check(X, W, A, B, where)
    _tensor(norm_w, "norm_w", (k,), X.dtype, X.device, where)
    _tensor(rstd, "rstd", (T,), torch.float32, X.device, where)
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        _tensor(dY[p], "d" + p.upper(), (T, n), X.dtype, X.device, where)
    o = dict(out or {})
    if need_dx and o.get("dX") is not None:
        _tensor(o["dX"], "dX", (T, k), X.dtype, X.device, where)
    _need(not accumulate_dx or (need_dx and o.get("dX") is not None),
          f"{where}: accumulate_dx needs out['dX']")
    for p, n in (("q", nq), ("k", nkv), ("v", nkv)):
        if o.get("dA_" + p) is not None:
            _tensor(o["dA_" + p], "dA_" + p, (r, k), X.dtype, X.device, where)
        if o.get("dB_" + p) is not None:
            _tensor(o["dB_" + p], "dB_" + p, (n, r), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    if need_dx and o.get("dX") is None:
        o["dX"] = torch.empty((T, k), dtype=X.dtype, device=X.device)
    if not need_dx:
        o["dX"] = None
    for p in ("q", "k", "v"):
        if o.get("dA_" + p) is None:
            o["dA_" + p] = torch.empty_like(A[p])
        if o.get("dB_" + p) is None:
            o["dB_" + p] = torch.empty_like(B[p])
    wsp, wsn = _workspace(OP_RMSNORM_QKV_BWD, dt, _wfmt(W["q"]), (T, k, nq, nkv, r), X.device,
                          workspace, False, stream)
    ws_ = [_wstruct(W[p]) for p in ("q", "k", "v")]
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate_dx else 0
    _check(lib().lora_rmsnorm_qkv_bwd(
        dt, T, k, nq, nkv, r, float(alpha), _ptr(X), _ptr(norm_w), _ptr(rstd),
        ctypes.byref(ws_[0]), _ptr(A["q"]), _ptr(B["q"]),
        ctypes.byref(ws_[1]), _ptr(A["k"]), _ptr(B["k"]),
        ctypes.byref(ws_[2]), _ptr(A["v"]), _ptr(B["v"]),
        _ptr(dY["q"]), _ptr(dY["k"]), _ptr(dY["v"]), _ptr(o["dX"]),
        _ptr(o["dA_q"]), _ptr(o["dB_q"]), _ptr(o["dA_k"]), _ptr(o["dB_k"]),
        _ptr(o["dA_v"]), _ptr(o["dB_v"]), flags, wsp, wsn, _stream(stream)), where)
    return o


def lora_merge(W: Weight, A, B, alpha: float, sign: int = 1, out=None, stream=None):
    """W + sign * (alpha/r) B A as a new [n, k] tensor (bf16 for 4-bit W)."""
    torch = _torch()
    where = "lora_merge"
    _need(isinstance(A, torch.Tensor) and A.dim() == 2, f"{where}: A must be a 2-D tensor")
    r, k = A.shape
    n = W.n if isinstance(W, Q4Weight) else W.shape[0]
    dt = _dtype_code(A)
    _weight(W, "W", n, k, A.dtype, A.device, where)
    _adapter(A, B, n, k, r, A.dtype, A.device, where)
    if out is not None:
        _tensor(out, "out", (n, k), A.dtype, A.device, where)
    _on_gpu(A, where)
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
    where = "lora_dequant4"
    _need(isinstance(q, Q4Weight) and not q.double_quant,
          f"{where}: needs a plain 4-bit weight (lora_decode_weight takes both forms)")
    dev = q.codes.device
    _weight(q, "W", q.n, q.k, torch.bfloat16, dev, where)
    if out is not None:
        _tensor(out, "out", (q.n, q.k), torch.bfloat16, dev, where)
    _on_gpu(q.codes, where)
    if out is None:
        out = torch.empty((q.n, q.k), dtype=torch.bfloat16, device=dev)
    _check(lib().lora_dequant4(q.n, q.k, _ptr(q.codes), _ptr(q.absmax), _ptr(q.codebook),
                               q.blocksize, LORA_BF16, _ptr(out), _stream(stream)),
           "lora_dequant4")
    return out


def lora_rmsnorm_fwd(X, w, eps: float, Y=None, rstd=None, stream=None):
    """RMSNorm of the rows of X: returns (Y, rstd) with rstd [T] fp32."""
    torch = _torch()
    where = "lora_rmsnorm_fwd"
    T, d = _x(X, where)
    _tensor(w, "w", (d,), X.dtype, X.device, where)
    if Y is not None:
        _tensor(Y, "Y", (T, d), X.dtype, X.device, where)
        _need(Y.data_ptr() != X.data_ptr(), f"{where}: Y may not alias X")
    if rstd is not None:
        _tensor(rstd, "rstd", (T,), torch.float32, X.device, where)
    _on_gpu(X, where)
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
    where = "lora_rmsnorm_bwd"
    T, d = _x(X, where)
    _tensor(w, "w", (d,), X.dtype, X.device, where)
    _tensor(rstd, "rstd", (T,), torch.float32, X.device, where)
    _tensor(dY, "dY", (T, d), X.dtype, X.device, where)
    if dX is None:
        _need(not accumulate, "accumulate needs dX")
    else:
        _tensor(dX, "dX", (T, d), X.dtype, X.device, where)
    _on_gpu(X, where)
    dt = _dtype_code(X)
    if dX is None:
        dX = torch.empty_like(X)
    flags = LORA_FLAG_ACCUMULATE_DX if accumulate else 0
    _check(lib().lora_rmsnorm_bwd(dt, T, d, _ptr(X), _ptr(w), _ptr(rstd), _ptr(dY), _ptr(dX),
                                  flags, _stream(stream)), "lora_rmsnorm_bwd")
    return dX


def lora_decode_weight(q: Q4Weight, out=None, stream=None):
    """Decode a 4-bit weight of either form (plain or double-quantised
    block constants) to a bf16 [n, k] tensor."""
    torch = _torch()
    where = "lora_decode_weight"
    _need(isinstance(q, Q4Weight), f"{where}: needs a 4-bit weight")
    dev = q.codes.device
    _weight(q, "W", q.n, q.k, torch.bfloat16, dev, where)
    if out is not None:
        _tensor(out, "out", (q.n, q.k), torch.bfloat16, dev, where)
    _on_gpu(q.codes, where)
    if out is None:
        out = torch.empty((q.n, q.k), dtype=torch.bfloat16, device=dev)
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
