"""Build liblora.so in-tree with hipcc for gfx950 (no GPU needed to build).

Also links liblora_timed.so: the same kernel objects with the host dispatch
file compiled with LORA_TIMING_HOOKS (include/liblora_timing.h), which the
benchmark loads to time one GEMM class inside a whole step."""
import os
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblora.so")
OUT_TIMED = os.path.join(HERE, "liblora_timed.so")
BUILD = os.path.join(HERE, "_build")
SOURCES = ["api.cpp", "gemm_nt.hip", "gemm_nt_q4.hip", "gemm_nn.hip", "gemm_nn_q4.hip",
           "gemm_nt_q4dq.hip", "gemm_nn_q4dq.hip"]
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC",
         "-I", os.path.join(ROOT, "include"), "-I", CSRC,
         # packed-fp32 VALU forms are kept out of every kernel
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops"]


def _hipcc():
    for c in (os.environ.get("HIPCC"), "/opt/rocm/bin/hipcc", "hipcc"):
        if c and (os.path.isabs(c) and os.path.exists(c) or not os.path.isabs(c)):
            return c
    return "hipcc"


def _compile(job):
    src, suffix, defs = job
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [_hipcc(), *FLAGS, *defs, "-x", "hip", "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
    return obj


def _link(out, objs):
    tmp = out + ".tmp"
    cmd = [_hipcc(), "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"link failed:\n{r.stderr[-4000:]}")
    os.replace(tmp, out)


def build(verbose=False):
    os.makedirs(BUILD, exist_ok=True)
    jobs_list = [(src, "", []) for src in SOURCES]
    jobs_list.append(("api.cpp", "_timed", ["-DLORA_TIMING_HOOKS"]))
    jobs = min(len(jobs_list), max(1, min(16, os.cpu_count() or 1)))
    with ThreadPoolExecutor(jobs) as ex:
        objs = list(ex.map(_compile, jobs_list))
    kernels = objs[1:len(SOURCES)]          # every object but the host dispatch file
    _link(OUT, [objs[0], *kernels])
    _link(OUT_TIMED, [objs[-1], *kernels])
    if verbose:
        print("built", OUT, "and", OUT_TIMED)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
