"""C-ABI contract tests that need no GPU: the library loads, exports every
symbol include/liblora.h declares, and rejects bad arguments before any HIP
call (so these calls are safe on a machine without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import lora_linear_fwd_amd as L

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "liblora.h")
TIMING_HEADER = os.path.join(ROOT, "include", "liblora_timing.h")

pytestmark = pytest.mark.skipif(not os.path.exists(L.LIB_PATH), reason="liblora not built")


def header_functions(path=HEADER):
    txt = open(path).read()
    txt = re.sub(r"/\*.*?\*/", "", txt, flags=re.S)
    return sorted(set(re.findall(r"\b(lora_[a-z0-9_]+)\s*\(", txt)))


def exported(path):
    out = subprocess.run(["nm", "-D", "--defined-only", path], capture_output=True,
                         text=True, check=True).stdout
    return set(re.findall(r"\bT\s+(lora_[a-z0-9_]+)$", out, flags=re.M))


def test_header_declares_the_entry_points():
    fns = header_functions()
    for name in ("lora_linear_fwd", "lora_linear_bwd", "lora_swiglu_mlp_fwd",
                 "lora_swiglu_mlp_bwd", "lora_dequant4", "lora_workspace_bytes",
                 "lora_strerror", "lora_abi_version", "lora_decode_weight", "lora_merge"):
        assert name in fns
    assert set(fns) == set(L.EXPORTS)


def test_library_exports_every_declared_symbol():
    assert set(header_functions()) <= exported(L.LIB_PATH)
    lib = L.lib()
    for name in header_functions():
        assert hasattr(lib, name)


def test_timing_hook_only_in_the_timing_build():
    # the production library carries no instrumentation state or symbol; the
    # benchmark's build exports everything liblora.h declares plus the hook
    timing = header_functions(TIMING_HEADER)
    assert timing == sorted(L.TIMING_EXPORTS)
    assert not set(timing) & exported(L.LIB_PATH)
    assert set(header_functions()) | set(timing) <= exported(L.TIMED_LIB_PATH)
    with pytest.raises(RuntimeError):
        L.time_next(L.KC_GATEUP_FWD, None, None)


def test_timing_build_has_the_same_kernels():
    # only the host dispatch object differs: every GPU kernel symbol is shared
    def kernels(path):
        out = subprocess.run(["nm", "--defined-only", path], capture_output=True, text=True,
                             check=True).stdout
        return set(re.findall(r"\s(_Z\S*k_\w+)$", out, flags=re.M))
    a, b = kernels(L.LIB_PATH), kernels(L.TIMED_LIB_PATH)
    assert a and a == b


def test_version_and_strerror():
    assert L.abi_version() == 4
    assert L.strerror(0) == "ok"
    for s in range(1, 7):
        assert L.strerror(s) and L.strerror(s) != "unknown status"
    assert L.strerror(99) == "unknown status"


def test_workspace_bytes_rules():
    wb = L.workspace_bytes
    assert wb(L.OP_LINEAR_FWD, L.LORA_BF16, 0, 8192, 4096, 4096, 16) > 0
    assert wb(L.OP_LINEAR_FWD, L.LORA_BF16, 0, 8192, 4096, 4096, 0) == 0
    assert wb(L.OP_LINEAR_FWD, L.LORA_BF16, 0, 8192, 4096, 4096, 129) == 0
    assert wb(L.OP_LINEAR_FWD, 7, 0, 8192, 4096, 4096, 16) == 0
    # MLP forward holds h [T x f] bf16 in the workspace
    assert wb(L.OP_MLP_FWD, L.LORA_BF16, 0, 8192, 4096, 14336, 16) >= 8192 * 14336 * 2
    # MLP backward holds de, dg
    assert wb(L.OP_MLP_BWD, L.LORA_BF16, 0, 8192, 4096, 14336, 16) >= 2 * 8192 * 14336 * 2
    assert wb(L.OP_LINEAR_BWD, L.LORA_F32, 0, 256, 512, 512, 8) == 2 * 256 * 8 * 4
    assert wb(L.OP_MLP_FWD | 0x200, L.LORA_BF16, 0, 8192, 4096, 14336, 16) == 0
    assert wb(L.OP_MLP_FWD, L.LORA_BF16, 5, 8192, 4096, 14336, 16) == 0
    # the double-quantised 4-bit form needs what the plain 4-bit form needs
    for op in (L.OP_LINEAR_FWD, L.OP_LINEAR_BWD, L.OP_MLP_FWD, L.OP_MLP_BWD):
        for m in (0, L.LORA_WS_MINIMAL):
            assert (wb(op | m, L.LORA_BF16, 2, 8192, 4096, 14336, 16)
                    == wb(op | m, L.LORA_BF16, 1, 8192, 4096, 14336, 16) > 0)


def test_weight_struct_layout_matches_header():
    """ctypes' lora_weight has the C struct's size and field offsets."""
    import tempfile
    fields = [f[0] for f in L.LoraWeightC._fields_]
    src = "#include <stddef.h>\n#include <stdio.h>\n#include \"liblora.h\"\nint main(void){"
    src += 'printf("%zu", sizeof(lora_weight));'
    src += "".join(f'printf(" %zu", offsetof(lora_weight, {f}));' for f in fields)
    src += "return 0;}\n"
    with tempfile.TemporaryDirectory() as d:
        c, exe = os.path.join(d, "layout.c"), os.path.join(d, "layout")
        open(c, "w").write(src)
        subprocess.run(["gcc", "-I", os.path.join(ROOT, "include"), c, "-o", exe], check=True)
        got = [int(v) for v in subprocess.run([exe], capture_output=True, text=True,
                                              check=True).stdout.split()]
    assert got[0] == ctypes.sizeof(L.LoraWeightC)
    assert got[1:] == [getattr(L.LoraWeightC, f).offset for f in fields]


def test_workspace_strategies():
    """The fast size adds exactly the weight copies to the minimal size."""
    wb, M = L.workspace_bytes, L.LORA_WS_MINIMAL
    T, d, f, r = 8192, 4096, 14336, 16
    # dense forwards copy nothing
    for op, kd, nf in ((L.OP_LINEAR_FWD, d, f), (L.OP_MLP_FWD, d, f)):
        assert wb(op, L.LORA_BF16, 0, T, kd, nf, r) == wb(op | M, L.LORA_BF16, 0, T, kd, nf, r)
    # 4-bit forwards hold decoded weights: W [n x k]; MLP Wg | Wu (Wd reuses it)
    assert (wb(L.OP_LINEAR_FWD, L.LORA_BF16, 1, T, d, f, r)
            - wb(L.OP_LINEAR_FWD | M, L.LORA_BF16, 1, T, d, f, r)) == f * d * 2
    # the MLP forward over decoded weights is the dense forward (its gate/up
    # epilogue forms h Ad^T) plus Wg | Wu; the minimal strategy's four-wave
    # gate/up GEMM leaves h Ad^T to a pass with smaller partials
    assert (wb(L.OP_MLP_FWD, L.LORA_BF16, 1, T, d, f, r)
            - wb(L.OP_MLP_FWD, L.LORA_BF16, 0, T, d, f, r)) == 2 * f * d * 2
    assert (wb(L.OP_MLP_FWD | M, L.LORA_BF16, 1, T, d, f, r)
            <= wb(L.OP_MLP_FWD, L.LORA_BF16, 0, T, d, f, r))
    # 4-bit backwards hold decoded, transposed weights: W^T; MLP [Wg^T | Wu^T]
    # (Wd^T reuses it); dense backwards read W in place in both strategies
    assert (wb(L.OP_LINEAR_BWD, L.LORA_BF16, 1, T, d, f, r)
            - wb(L.OP_LINEAR_BWD | M, L.LORA_BF16, 1, T, d, f, r)) == f * d * 2
    assert (wb(L.OP_MLP_BWD, L.LORA_BF16, 1, T, d, f, r)
            - wb(L.OP_MLP_BWD | M, L.LORA_BF16, 1, T, d, f, r)) == 2 * f * d * 2
    for op in (L.OP_LINEAR_BWD, L.OP_MLP_BWD):
        assert wb(op, L.LORA_BF16, 0, T, d, f, r) == wb(op | M, L.LORA_BF16, 0, T, d, f, r)
    # fp32 has one strategy
    assert wb(L.OP_MLP_BWD, L.LORA_F32, 0, 67, 48, 80, 5) == wb(L.OP_MLP_BWD | M, L.LORA_F32, 0, 67, 48, 80, 5)


# fake, aligned, non-null host addresses: every call below fails validation
# before touching them
_buf = (ctypes.c_uint8 * 4096)()
_base = (ctypes.addressof(_buf) + 255) & ~255
P = ctypes.c_void_p(_base)
P_MIS = ctypes.c_void_p(_base + 2)


def _w(fmt=0, blocksize=0, w=P, codes=None, absmax=None, codebook=None):
    return L.LoraWeightC(fmt, blocksize, w, codes, absmax, codebook)


def _wdq(codes=P, codebook=P, acodes=P, atable=P, ascale=P, abs2=256, blocksize=64):
    return L.LoraWeightC(2, blocksize, None, codes, None, codebook, acodes, atable, ascale, 0.04,
                         abs2)


def fwd(dtype=1, T=16, k=64, n=64, r=8, X=P, W=None, A=P, B=P, Y=P, ws=P, wsb=1 << 30):
    W = W or _w()
    return L.lib().lora_linear_fwd(dtype, T, k, n, r, 16.0, X, ctypes.byref(W), A, B, Y, ws,
                                   wsb, None)


def test_linear_fwd_validation_codes():
    assert fwd(X=None) == 1
    assert fwd(Y=None) == 1
    assert fwd(W=_w(w=None)) == 1
    assert fwd(k=60) == 2           # bf16 rows must be 16-byte multiples
    assert fwd(n=12) == 2
    assert fwd(T=-1) == 2
    assert fwd(k=0) == 2
    assert fwd(r=0) == 2
    assert fwd(r=129) == 3
    assert fwd(dtype=5) == 3
    assert fwd(X=P_MIS) == 5
    assert fwd(wsb=0) == 4
    assert fwd(ws=None) == 1
    # 4-bit weights: bf16 only, blocksize 64, k % 64 == 0, all three pointers
    q4 = _w(1, 64, None, P, P, P)
    assert fwd(dtype=0, W=q4) == 3
    assert fwd(W=_w(1, 32, None, P, P, P)) == 3
    assert fwd(k=72, W=q4) == 2
    assert fwd(W=_w(1, 64, None, P, None, P)) == 1
    assert fwd(W=_w(7)) == 3
    # double-quantised constants: bf16, second-level block 256, every pointer
    assert fwd(dtype=0, W=_wdq()) == 3
    assert fwd(W=_wdq(abs2=128)) == 3
    assert fwd(W=_wdq(blocksize=32)) == 3
    assert fwd(W=_wdq(acodes=None)) == 1
    assert fwd(W=_wdq(atable=None)) == 1
    assert fwd(W=_wdq(ascale=None)) == 1
    assert fwd(W=_wdq(codebook=None)) == 1
    assert fwd(W=_wdq(ascale=P_MIS)) == 5
    assert fwd(W=_wdq(acodes=P_MIS)) == 5
    assert fwd(k=72, W=_wdq()) == 2


def test_linear_bwd_validation_codes():
    W = _w()
    call = lambda **kw: L.lib().lora_linear_bwd(
        kw.get("dtype", 1), 16, 64, 64, 8, 16.0, P, ctypes.byref(W), P, P, kw.get("dY", P),
        kw.get("dX", P), kw.get("dA", P), kw.get("dB", P), kw.get("flags", 0), P, 1 << 30, None)
    assert call(dY=None) == 1
    assert call(dA=None) == 1
    assert call(dX=P_MIS) == 5
    assert call(flags=2) == 3


def test_mlp_validation_codes():
    W = _w()
    args = lambda **kw: [1, kw.get("T", 16), kw.get("d", 64), kw.get("f", 128), 8, 16.0, P,
                         ctypes.byref(W), P, P, ctypes.byref(W), P, P, ctypes.byref(W), P, P]
    lib = L.lib()
    assert lib.lora_swiglu_mlp_fwd(*args(d=60), P, P, P, P, 1 << 30, None) == 2
    assert lib.lora_swiglu_mlp_fwd(*args(), None, P, P, P, 1 << 30, None) == 1
    assert lib.lora_swiglu_mlp_fwd(*args(), P, P, P, P, 10, None) == 4
    assert lib.lora_swiglu_mlp_bwd(*args(), P, P, P, P, P, P, P, P, None, P, P, 1 << 30,
                                   None) == 1
    q4 = _w(1, 64, None, P, P, P)
    mixed = [1, 16, 64, 128, 8, 16.0, P, ctypes.byref(q4), P, P, ctypes.byref(W), P, P,
             ctypes.byref(W), P, P]
    assert lib.lora_swiglu_mlp_fwd(*mixed, P, P, P, P, 1 << 30, None) == 3
    # gate and up share one format (the fused gate/up GEMM reads both alike)
    dq = _wdq()
    mixed = [1, 16, 64, 128, 8, 16.0, P, ctypes.byref(q4), P, P, ctypes.byref(dq), P, P,
             ctypes.byref(dq), P, P]
    assert lib.lora_swiglu_mlp_fwd(*mixed, P, P, P, P, 1 << 30, None) == 3


def test_decode_weight_validation_codes():
    lib = L.lib()
    dq, q4 = _wdq(), _w(1, 64, None, P, P, P)
    call = lambda W, n=16, k=128, dt=1, out=P: lib.lora_decode_weight(n, k, ctypes.byref(W), dt,
                                                                      out, None)
    assert call(_w()) == 3                 # dense weights have nothing to decode
    assert call(dq, out=None) == 1
    assert call(q4, dt=0) == 3
    assert call(dq, k=100) == 2
    assert call(dq, n=0) == 2
    assert call(_wdq(abs2=64)) == 3
    assert call(q4, out=P_MIS) == 5
    assert lib.lora_decode_weight(16, 128, None, 1, P, None) == 1


def test_dequant4_validation_codes():
    lib = L.lib()
    assert lib.lora_dequant4(16, 128, None, P, P, 64, 1, P, None) == 1
    assert lib.lora_dequant4(16, 100, P, P, P, 64, 1, P, None) == 2
    assert lib.lora_dequant4(16, 128, P, P, P, 32, 1, P, None) == 3
    assert lib.lora_dequant4(16, 128, P, P, P, 64, 0, P, None) == 3
    assert lib.lora_dequant4(16, 128, P_MIS, P, P, 64, 1, P, None) == 5


def test_merge_validation_codes():
    W = _w()
    call = lambda **kw: L.lib().lora_merge(kw.get("dtype", 1), kw.get("n", 64), kw.get("k", 64),
                                          kw.get("r", 8), 16.0, kw.get("sign", 1),
                                          ctypes.byref(kw.get("W", W)), kw.get("A", P),
                                          kw.get("B", P), kw.get("out", P), None)
    assert call(A=None) == 1
    assert call(out=None) == 1
    assert call(W=_w(w=None)) == 1
    assert call(dtype=4) == 3
    assert call(sign=0) == 3
    assert call(n=0) == 2
    assert call(k=-1) == 2
    assert call(r=129) == 3
    assert call(out=P_MIS) == 5
    assert call(dtype=0, W=_w(1, 64, None, P, P, P)) == 3     # 4-bit is bf16-only
    assert call(k=72, W=_w(1, 64, None, P, P, P)) == 2        # 4-bit needs k % 64 == 0


def test_rmsnorm_validation_codes():
    lib = L.lib()
    fwd = lambda dt=1, T=16, d=64, eps=1e-5, X=P, w=P, Y=P, r=P: lib.lora_rmsnorm_fwd(
        dt, T, d, eps, X, w, Y, r, None)
    assert fwd(dt=3) == 3
    assert fwd(eps=-1.0) == 3
    assert fwd(eps=float("nan")) == 3
    assert fwd(eps=float("inf")) == 3
    assert fwd(d=60) == 2            # bf16 rows are 16-byte multiples
    assert fwd(d=0) == 2
    assert fwd(T=-1) == 2
    assert fwd(w=None) == 1
    assert fwd(X=None) == 1
    assert fwd(r=None) == 1
    assert fwd(Y=P_MIS) == 5
    assert fwd(T=0, X=None, Y=None, r=None) == 0     # nothing to do, nothing launched
    bwd = lambda dt=1, T=16, d=64, flags=0, dY=P, dX=P: lib.lora_rmsnorm_bwd(
        dt, T, d, P, P, P, dY, dX, flags, None)
    assert bwd(flags=2) == 3
    assert bwd(dY=None) == 1
    assert bwd(dX=P_MIS) == 5
    assert bwd(dt=0, d=60, dX=None) == 1   # fp32 takes any width: the null dX is what fails


def test_feature_size_limit():
    # feature sizes up to 2^20: a GEMM tile's 256 rows then span < 2^31 bytes
    # (one buffer descriptor); larger sizes are refused before any HIP call
    assert fwd(k=(1 << 20) + 8) == 2
    assert fwd(n=(1 << 20) + 8) == 2
    W = _w()
    args = [1, 16, 64, (1 << 20) + 64, 8, 16.0, P, ctypes.byref(W), P, P, ctypes.byref(W), P, P,
            ctypes.byref(W), P, P]
    assert L.lib().lora_swiglu_mlp_fwd(*args, P, P, P, P, 1 << 40, None) == 2


def test_grid_size_limits():
    # 2^30 tokens by 2^24 features would need more than 2^31 GEMM tiles
    assert fwd(T=1 << 30, k=64, n=1 << 24) == 2
    lib = L.lib()
    assert lib.lora_decode_weight(1 << 24, 1 << 24, ctypes.byref(_w(1, 64, None, P, P, P)), 1, P,
                                  None) == 2
    assert lib.lora_dequant4(1 << 24, 1 << 24, P, P, P, 64, 1, P, None) == 2


def test_noalloc_validation_before_any_hip_call():
    # the allocation-free linear backward checks its arguments, then the size
    # of its static scratch array, before it touches the GPU
    lib = L.lib()
    W = _w()
    call = lambda T=16, k=64, n=64, r=8, **kw: lib.lora_linear_bwd_noalloc(
        kw.get("dtype", 1), T, k, n, r, 16.0, kw.get("X", P), ctypes.byref(W), P, P,
        kw.get("dY", P), kw.get("dX", P), kw.get("dA", P), P, kw.get("flags", 0), None)
    assert call(dY=None) == 1
    assert call(dA=None) == 1
    assert call(dX=P_MIS) == 5
    assert call(k=60) == 2
    assert call(r=129) == 3
    assert call(flags=2) == 3
    big = L.workspace_bytes(L.OP_LINEAR_BWD | L.LORA_WS_MINIMAL, 1, 0, 65536, 4096, 4096, 128)
    assert big > L.LORA_NOALLOC_SCRATCH_BYTES
    assert call(T=65536, k=4096, n=4096, r=128) == 4


def test_fused_norm_validation_codes():
    lib = L.lib()
    W = _w()
    q4 = _w(1, 64, None, P, P, P)
    def fwd_(dtype=1, eps=1e-5, nw=P, rstd=P, Wg=W, wsb=1 << 30):
        return lib.lora_rmsnorm_swiglu_mlp_fwd(dtype, 16, 64, 128, 8, 16.0, eps, P, nw,
                                               ctypes.byref(Wg), P, P, ctypes.byref(Wg), P, P,
                                               ctypes.byref(W), P, P, P, P, P, rstd, P, wsb, None)
    assert fwd_(nw=None) == 1
    assert fwd_(rstd=None) == 1
    assert fwd_(dtype=0) == 3           # bf16 only
    assert fwd_(Wg=q4) == 3             # a 4-bit weight cannot hold W diag(w)
    assert fwd_(eps=-1.0) == 3
    assert fwd_(eps=float("nan")) == 3
    assert fwd_(wsb=16) == 4
    def bwd_(flags=0, rstd=P):
        return lib.lora_rmsnorm_swiglu_mlp_bwd(1, 16, 64, 128, 8, 16.0, P, P, rstd,
                                               ctypes.byref(W), P, P, ctypes.byref(W), P, P,
                                               ctypes.byref(W), P, P, P, P, P, P,
                                               P, P, P, P, P, P, flags, P, 1 << 30, None)
    assert bwd_(flags=2) == 3
    assert bwd_(rstd=None) == 1
    # the fused backward needs room for the per-row partials of the norm
    assert L.workspace_bytes(L.OP_RMSNORM_MLP_BWD, 1, 0, 8192, 4096, 14336, 16) > \
        L.workspace_bytes(L.OP_MLP_BWD, 1, 0, 8192, 4096, 14336, 16)
    assert L.workspace_bytes(L.OP_RMSNORM_MLP_FWD, 1, 1, 8192, 4096, 14336, 16) == 0
    assert L.workspace_bytes(L.OP_RMSNORM_MLP_FWD, 0, 0, 8192, 4096, 14336, 16) == 0
    assert lib.lora_fold_norm_weight(1, 16, 60, P, P, P, None) == 2
    assert lib.lora_fold_norm_weight(0, 16, 64, P, P, P, None) == 3
    assert lib.lora_fold_norm_weight(1, 16, 64, P, None, P, None) == 1


def test_fused_norm_qkv_validation_codes():
    lib = L.lib()
    W = _w()
    q4 = _w(1, 64, None, P, P, P)
    def fwd_(dtype=1, k=64, nq=256, nkv=256, r=8, eps=1e-5, nw=P, rstd=P, Wq=W, wsb=1 << 30):
        return lib.lora_rmsnorm_qkv_fwd(dtype, 16, k, nq, nkv, r, 16.0, eps, P, nw,
                                        ctypes.byref(Wq), P, P, ctypes.byref(W), P, P,
                                        ctypes.byref(W), P, P, P, P, P, rstd, P, wsb, None)
    assert fwd_(nw=None) == 1
    assert fwd_(rstd=None) == 1
    assert fwd_(dtype=0) == 3           # bf16 only
    assert fwd_(Wq=q4) == 3             # a 4-bit weight cannot hold W diag(w)
    assert fwd_(nkv=136) == 3           # the stacked GEMM's shapes only
    assert fwd_(r=100) == 3             # 3r > 256
    assert fwd_(k=60) == 2
    assert fwd_(eps=float("inf")) == 3
    assert fwd_(wsb=16) == 4
    def bwd_(flags=0, rstd=P, dA=P):
        return lib.lora_rmsnorm_qkv_bwd(1, 16, 64, 256, 256, 8, 16.0, P, P, rstd,
                                        ctypes.byref(W), P, P, ctypes.byref(W), P, P,
                                        ctypes.byref(W), P, P, P, P, P, P,
                                        dA, P, P, P, P, P, flags, P, 1 << 30, None)
    assert bwd_(flags=2) == 3
    assert bwd_(rstd=None) == 1
    assert bwd_(dA=None) == 1
    ws = lambda op, dt=1, fmt=0, nkv=1024: int(lib.lora_qkv_workspace_bytes(op, dt, fmt, 8192, 4096,
                                                                          4096, nkv, 16))
    # the fused backward keeps the projections' input gradient for the row pass
    assert ws(L.OP_RMSNORM_QKV_BWD) == ws(L.OP_QKV_BWD) + 8192 * 4096 * 2
    assert ws(L.OP_RMSNORM_QKV_FWD) == ws(L.OP_QKV_FWD)
    assert ws(L.OP_RMSNORM_QKV_FWD, fmt=1) == 0
    assert ws(L.OP_RMSNORM_QKV_FWD, dt=0) == 0
    assert ws(L.OP_RMSNORM_QKV_BWD, nkv=1000) == 0
