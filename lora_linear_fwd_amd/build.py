"""Build liblora.so in-tree with hipcc for gfx950 (no GPU needed to build).

Also links liblora_timed.so: the same kernel objects with the host dispatch
file compiled with LORA_TIMING_HOOKS (include/liblora_timing.h), which the
benchmark loads to time one GEMM class inside a whole step."""
import os
import re
import subprocess
import sys
from concurrent.futures import ThreadPoolExecutor

HERE = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(HERE)
CSRC = os.path.join(HERE, "csrc")
OUT = os.path.join(HERE, "liblora.so")
OUT_TIMED = os.path.join(HERE, "liblora_timed.so")
# per-kernel register / scratch use, from the compiler's resource remarks
RESOURCE_REPORT = os.path.join(HERE, "_build", "kernel_resources.txt")
# kernels that must not touch scratch memory: a register spill in the GEMM
# main loop costs several-fold (measured: 0.72 -> 3.6 ms for one GEMM)
NO_SPILL = re.compile(r"k_lora_gemm_pp")
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


def _resources(stderr):
    """{kernel: {field: value}} from -Rpass-analysis=kernel-resource-usage."""
    out, cur = {}, None
    for line in stderr.splitlines():
        m = re.search(r"remark: Function Name: (\S+)", line)
        if m:
            cur = out.setdefault(m.group(1), {})
            continue
        m = re.search(r"remark:\s+([A-Za-z /\[\]]+?):\s*(\S+) \[-Rpass-analysis", line)
        if m and cur is not None:
            cur[m.group(1).strip()] = m.group(2)
    return out


def _compile(job):
    src, suffix, defs = job
    obj = os.path.join(BUILD, os.path.splitext(src)[0] + suffix + ".o")
    cmd = [_hipcc(), *FLAGS, *defs, "-Rpass-analysis=kernel-resource-usage", "-x", "hip", "-c",
           os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed for {src}:\n{r.stderr[-4000:]}")
    return obj, _resources(r.stderr)


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
        results = list(ex.map(_compile, jobs_list))
    objs = [o for o, _ in results]
    res = {}
    for _, r in results:
        res.update(r)
    with open(RESOURCE_REPORT, "w") as fh:
        for k in sorted(res):
            fh.write(k + " " + " ".join(f"{f.replace(' ', '_')}={v}" for f, v in res[k].items())
                     + "\n")
    spills = [k for k, v in res.items()
              if NO_SPILL.search(k) and (v.get("ScratchSize [bytes/lane]", "0") != "0"
                                         or v.get("VGPRs Spill", "0") != "0")]
    if spills:
        raise RuntimeError("GEMM kernels use scratch memory (register spills): " + ", ".join(spills)
                           + f"; see {RESOURCE_REPORT}")
    kernels = objs[1:len(SOURCES)]          # every object but the host dispatch file
    _link(OUT, [objs[0], *kernels])
    _link(OUT_TIMED, [objs[-1], *kernels])
    if verbose:
        print("built", OUT, "and", OUT_TIMED)
    return OUT


if __name__ == "__main__":
    build(verbose=True)
    sys.exit(0)
