"""Throughput of the LoRA-SwiGLU MLP forward + hand-derived backward on one GPU.

One step = lora_swiglu_mlp_fwd + lora_swiglu_mlp_bwd (with dX) over one batch
of synthetic, seeded inputs already resident in HBM; default workload is the
Llama-3-8B MLP shape (T = 4 x 2048 tokens, d = 4096, f = 14336, LoRA r = 16,
alpha = 16 on gate, up and down; bf16 storage, fp32 accumulation).

Prints ONE JSON line.  `value` is algorithmic TFLOP/s
(12 T d f + 18 T r (d + f) FLOP per step); tokens/s and percent of the
MI355X bf16 dense MFMA peak ride along.  The roofline object describes the
slowest GEMM of the step, timed with HIP events recorded by the library on
its own launch stream around every launch of that kernel in the timed
region.  cpu_baseline runs the float64 CPU oracle on a bounded sample of the
same workload (fewer tokens).
"""
import argparse
import json
import os
import sys
import time

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6        # 256 CU x 2.4 GHz x 4096 flop/clk/CU (dense)
PEAK_HBM_GBS = 8000.0
CSRC = os.path.join(ROOT, "lora_linear_fwd_amd", "csrc")
TRAFFIC_SUMMARY = os.path.join(ROOT, "profiles", "gemm_{shape}_hbm_traffic.md")
KC_NAMES = ["gate/up fwd GEMM + SwiGLU epilogue", "down fwd GEMM",
            "down bwd GEMM + SwiGLU' epilogue", "gate/up bwd dX GEMM"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=20)
    ap.add_argument("--warmup", type=int, default=5)
    ap.add_argument("--config", type=int, default=3, choices=(2, 3, 4, 5),
                    help="2, 3, 5: LoRA-SwiGLU MLP; 4: q/k/v/o LoRA projections + MLP")
    ap.add_argument("--qkv-separate", action="store_true",
                    help="config 4: run q, k, v as three LoRA linears instead of the fused call")
    ap.add_argument("--dq", action="store_true",
                    help="workload 5 with double-quantised 4-bit block constants")
    ap.add_argument("--minimal-ws", action="store_true",
                    help="minimal workspace (no weight copies; 4-bit decoded inside the GEMMs)")
    ap.add_argument("--weights-as-stored", action="store_true",
                    help="dense weights without a caller-kept transpose (the backward dX GEMMs "
                         "then read W as stored); default: W^T is kept next to each frozen W")
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--cpu-tokens", type=int, default=8192,
                    help="tokens of the workload the CPU oracle baseline runs on")
    ap.add_argument("--calibrate-copy", action="store_true",
                    help="only run a 256 MiB device-to-device copy (3 times): the "
                         "known-size reference for the FETCH_SIZE / WRITE_SIZE counters")
    ap.add_argument("--summarize-counters", nargs=4, metavar=("FETCH_CSV", "WRITE_CSV",
                                                              "COPY_FETCH_CSV", "COPY_WRITE_CSV"),
                    help="print the HBM-traffic summary (markdown) of the GEMM classes from "
                         "rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE counter_collection CSVs of "
                         "bench.py and of --calibrate-copy")
    ap.add_argument("--with-trace", nargs=2, metavar=("TRACE_DIR", "STEP"),
                    help="with --summarize-counters: durations from one step of a rocprofv3 "
                         "--kernel-trace output folder of the same workload, and HBM rates")
    ap.add_argument("--summarize-sq", nargs=2, metavar=("SQ_CSV_1", "SQ_CSV_2"),
                    help="print the GEMM classes' shader-engine counter table from the two "
                         "rocprofv3 --pmc counter_collection CSVs of bench.py")
    ap.add_argument("--summarize-trace", nargs=2, metavar=("TRACE_DIR", "STEP"),
                    help="print the kernel table and one step's dispatches from a "
                         "rocprofv3 --kernel-trace --stats output folder of bench.py")
    return ap.parse_args()


def kernel_source_digest():
    """sha256 over the HIP sources (any change invalidates stored counters)."""
    import hashlib
    h = hashlib.sha256()
    for name in sorted(os.listdir(CSRC)):
        with open(os.path.join(CSRC, name), "rb") as fh:
            h.update(name.encode() + b"\0" + fh.read())
    return h.hexdigest()


def _counter_rows(path):
    import csv
    rows = []
    with open(path) as fh:
        for r in csv.DictReader(fh):
            rows.append((int(r["Dispatch_Id"]), r["Kernel_Name"], float(r["Counter_Value"])))
    rows.sort()
    return rows


# A profiled `bench.py --steps 1 --warmup 1` runs the step form that `value`
# times in its first five steps (warm-up, two probe steps, the timed step, the
# per-class pass); later passes use other forms (weights as stored, the norm
# comparisons).  Summaries average steps 2-5 of the run.
PROFILED_STEPS = range(1, 5)


def _step_starts(names):
    """Index of each step's first dispatch.  The forward opens with the
    rank-r pass over X (width 2r = 32 for the MLP workloads, 3r = 192 for the
    attention workload's fused q/k/v) or the norm's rstd pass, preceded by
    the operand copies (k_prep) where the call makes them, and by the 4-bit
    decodes of the gate and up weights when it has them.  (In the MLP
    backward the 32-wide pass over X follows a reduction, never k_prep.)"""
    out = []
    for i in range(len(names) - 1):
        opener = ("k_skinny_nt<32" in names[i + 1] or "k_skinny_nt<192" in names[i + 1]
                  or "k_rmsnorm_fwd" in names[i + 1])
        if "k_prep" in names[i] and opener:
            j = i
        elif ("k_skinny_nt<32" in names[i] and (i == 0 or not any(
                k in names[i - 1] for k in ("k_reduce_side", "k_prep")))):
            j = i
        else:
            continue
        while j > 0 and "k_dequant4(" in names[j - 1]:
            j -= 1
        out.append(j)
    return out


def _steps(rows):
    """rows sorted by dispatch -> list of steps, each a list of rows."""
    names = [r[1] for r in rows]
    st = _step_starts(names) + [len(rows)]
    return [rows[st[i]:st[i + 1]] for i in range(len(st) - 1)]


def _gemm_class_values(rows):
    """Counter value (KiB) per dispatch of each GEMM class over the profiled
    steps: a step launches the GEMMs in the order gate/up fwd, down fwd,
    down bwd, gate/up bwd."""
    out = {i: [] for i in range(4)}
    steps = _steps(rows)
    for k in PROFILED_STEPS:
        gem = [v for _, name, v in steps[k] if "k_lora_gemm" in name]
        assert len(gem) == 4, f"step {k}: {len(gem)} GEMM dispatches"
        for j, v in enumerate(gem):
            out[j].append(v)
    return out


def _short(name, width=72):
    name = name.replace("lora::", "").replace("void ", "")
    return name if len(name) <= width else name[:width - 3] + "..."


def traffic_path(cfg):
    from lora_inputs import CONFIGS
    c = CONFIGS[cfg]
    shape = "T%d_d%d_f%d_r%d" % (c["T"], c["d"], c["f"], c["r"])
    return TRAFFIC_SUMMARY.format(shape=shape + ("_q4" if c.get("q4") else ""))


def _trace_rows(trace_dir):
    import csv
    tr = sorted(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))),
                key=lambda r: int(r["Start_Timestamp"]))
    return [(int(r["Start_Timestamp"]), r["Kernel_Name"], int(r["End_Timestamp"])) for r in tr]


def _longest_runs(names):
    """name -> (start, length) of its longest run of consecutive dispatches."""
    out, i = {}, 0
    while i < len(names):
        j = i
        while j < len(names) and names[j] == names[i]:
            j += 1
        if j - i > out.get(names[i], (0, 0))[1]:
            out[names[i]] = (i, j - i)
        i = j
    return out


def summarize_counters(fetch_csv, write_csv, cf_csv, cw_csv, cfg, trace=None):
    """Markdown summary with a machine-readable line read back by bench.py:
    per GEMM class and, for one step, per dispatch.  With trace = (folder of
    a kernel trace of the same workload, step index), each dispatch also gets
    its traced duration and the HBM rate of its counted bytes, and kernels
    launched in timing loops of their own (RMSNorm) get a row each."""
    import statistics
    copy_bytes = 256 << 20
    cf = [v for _, n, v in _counter_rows(cf_csv) if "copyBuffer" in n]
    cw = [v for _, n, v in _counter_rows(cw_csv) if "copyBuffer" in n]
    f_fac = copy_bytes / (sum(cf) / len(cf) * 1024)
    w_fac = copy_bytes / (sum(cw) / len(cw) * 1024)
    frows, wrows = _counter_rows(fetch_csv), _counter_rows(write_csv)
    fv, wv = _gemm_class_values(frows), _gemm_class_values(wrows)
    per = {}
    for i in range(4):
        fb = sum(fv[i]) / len(fv[i]) * 1024 * f_fac
        wb = sum(wv[i]) / len(wv[i]) * 1024 * w_fac
        per[KC_NAMES[i]] = {"fetch_bytes": round(fb), "write_bytes": round(wb),
                            "traffic_bytes": round(fb + wb)}
    rec = {"config_id": cfg, "source_sha256": kernel_source_digest(),
           "fetch_scale": round(f_fac, 4), "write_scale": round(w_fac, 4), "per_launch": per}
    lines = ["| GEMM | FETCH (scaled) MB | WRITE (scaled) MB | total MB |", "|---|---|---|---|"]
    for k, v in per.items():
        lines.append(f"| {k} | {v['fetch_bytes'] / 1e6:.1f} | {v['write_bytes'] / 1e6:.1f} | "
                     f"{v['traffic_bytes'] / 1e6:.1f} |")
    k = PROFILED_STEPS[0]
    fs, ws = _steps(frows)[k], _steps(wrows)[k]
    durs = None
    if trace is not None:
        tsteps = _steps(_trace_rows(trace[0]))
        tstep = tsteps[int(trace[1])]
        assert [n for _, n, _ in tstep] == [n for _, n, _ in fs], "trace step differs"
        durs = [(e - b) / 1e3 for b, _, e in tstep]
    head = "| # | kernel | FETCH MB | WRITE MB |"
    if durs:
        head += " us | GB/s | of 8 TB/s |"
    lines += ["", f"Every dispatch of step {k + 1} (scaled MB" +
              (f"; duration from step {int(trace[1]) + 1} of the kernel trace" if durs else "") +
              "):", "", head, "|---" * (head.count("|") - 1) + "|"]
    for i, ((_, n, fv_), (_, n2, wv_)) in enumerate(zip(fs, ws)):
        assert n == n2, (n, n2)
        fb, wb = fv_ * 1024 * f_fac, wv_ * 1024 * w_fac
        row = f"| {i} | `{_short(n)}` | {fb / 1e6:.1f} | {wb / 1e6:.1f} |"
        if durs:
            gbs = (fb + wb) / (durs[i] * 1e-6) / 1e9
            row += f" {durs[i]:.1f} | {gbs:.0f} | {gbs / PEAK_HBM_GBS:.2f} |"
        lines.append(row)
    if durs:
        fn, wn = [n for _, n, _ in frows], [n for _, n, _ in wrows]
        tr = _trace_rows(trace[0])
        tn = [n for _, n, _ in tr]
        fr, wr, trr = _longest_runs(fn), _longest_runs(wn), _longest_runs(tn)
        loops = [n for n, (_, ln) in fr.items() if ln >= 10 and "k_lora_gemm" not in n]
        if loops:
            lines += ["", "Kernels launched in timing loops of their own (medians over the "
                      "longest run of consecutive dispatches of each):", "",
                      "| kernel | dispatches | FETCH MB | WRITE MB | us | GB/s | of 8 TB/s |",
                      "|---|---|---|---|---|---|---|"]
            for n in loops:
                (a0, la), (b0, lb), (c0, lc) = fr[n], wr[n], trr[n]
                fb = statistics.median(v for _, _, v in frows[a0:a0 + la]) * 1024 * f_fac
                wb = statistics.median(v for _, _, v in wrows[b0:b0 + lb]) * 1024 * w_fac
                us = statistics.median((e - b) / 1e3 for b, _, e in tr[c0:c0 + lc])
                gbs = (fb + wb) / (us * 1e-6) / 1e9
                lines.append(f"| `{_short(n)}` | {la} | {fb / 1e6:.1f} | {wb / 1e6:.1f} | "
                             f"{us:.1f} | {gbs:.0f} | {gbs / PEAK_HBM_GBS:.2f} |")
    return "\n".join(lines) + "\n\ntraffic-record: " + json.dumps(rec) + "\n"


def summarize_sq(csv1, csv2):
    """Shader-engine counters of the four GEMM classes (medians over the
    profiled steps) from two --pmc runs: clock, achieved MFMA rate, MFMA-busy
    fraction, LDS bank conflicts and the share of wave time waiting on LDS."""
    import csv
    import statistics

    def load(path):
        rows = {}
        for r in csv.DictReader(open(path)):
            key = (int(r["Dispatch_Id"]), r["Kernel_Name"])
            dur = (int(r["End_Timestamp"]) - int(r["Start_Timestamp"])) * 1e-9
            rows.setdefault(key, {"dur": dur})[r["Counter_Name"]] = float(r["Counter_Value"])
        disp = sorted(rows)
        steps = _steps([(i, n, 0.0) for i, n in disp])
        out = {i: [] for i in range(4)}
        for k in PROFILED_STEPS:
            gem = [(i, n) for i, n, _ in steps[k] if "k_lora_gemm" in n]
            assert len(gem) == 4
            for j, key in enumerate(gem):
                out[j].append(rows[key])
        return out

    a, b = load(csv1), load(csv2)
    med = statistics.median
    lines = ["| GEMM | dispatches | duration ms | clock GHz | TFLOP/s | peak at that clock "
             "| MFMA busy | LDS bank conflicts | wave time waiting on LDS issue |",
             "|---|---|---|---|---|---|---|---|---|"]
    for i in range(4):
        A, B = a[i], b[i]
        clk = med([x["GRBM_GUI_ACTIVE"] / 8 / x["dur"] for x in B])   # one GRBM per XCD
        dur = med([x["dur"] for x in B])
        tf = med([x["SQ_INSTS_VALU_MFMA_MOPS_BF16"] * 512 / x["dur"] for x in A]) / 1e12
        busy = med([x["SQ_VALU_MFMA_BUSY_CYCLES"] / 1024 / (clk * x["dur"]) for x in A])
        bc = med([x["SQ_LDS_BANK_CONFLICT"] for x in A])
        wl = med([x["SQ_WAIT_INST_LDS"] / x["SQ_WAVE_CYCLES"] for x in A])
        lines.append(f"| {KC_NAMES[i]} | {len(B)} | {dur * 1e3:.3f} | {clk / 1e9:.2f} | "
                     f"{tf:.0f} | {256 * 4096 * clk / 1e12:.0f} | {busy * 100:.0f} % | "
                     f"{bc:.0f} | {wl * 100:.1f} % |")
    return "\n".join(lines) + "\n"


def summarize_trace(trace_dir, step):
    """rocprofv3 --kernel-trace --stats output of a bench.py run: the stats
    table as written, and every dispatch of step `step` (0-based) with its
    start offset, the gap before it and its duration."""
    import csv
    stats = list(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_stats.csv"))))
    lines = ["| kernel | calls | avg us | min us | max us | % of GPU time |",
             "|---|---|---|---|---|---|"]
    for r in stats:
        if "copyBuffer" in r["Name"]:
            continue
        lines.append(f"| `{_short(r['Name'])}` | {r['Calls']} | {float(r['AverageNs']) / 1e3:.1f} "
                     f"| {float(r['MinNs']) / 1e3:.1f} | {float(r['MaxNs']) / 1e3:.1f} | "
                     f"{float(r['Percentage']):.2f} |")
    tr = sorted(csv.DictReader(open(os.path.join(trace_dir, "run_kernel_trace.csv"))),
                key=lambda r: int(r["Start_Timestamp"]))
    rows = [(int(r["Start_Timestamp"]), r["Kernel_Name"], int(r["End_Timestamp"])) for r in tr]
    steps = _steps(rows)
    one = steps[step]
    t0 = prev = one[0][0]
    lines += ["", f"Step {step + 1} of {len(steps)} found in the trace (offset / gap before / "
                  "duration, us):", "", "```"]
    for s, n, e in one:
        lines.append(f"{(s - t0) / 1e3:8.1f} gap {max(0, s - prev) / 1e3:5.1f} "
                     f"dur {(e - s) / 1e3:8.1f}  {_short(n, 64)}")
        prev = e
    lines += [f"step span {(prev - t0) / 1e3:.1f} us", "```"]
    return "\n".join(lines) + "\n"


def stored_traffic(cfg, kernel_name):
    """HBM bytes per launch of `kernel_name` from the committed counter
    summary, or None when there is none or the HIP sources changed since."""
    from lora_inputs import CONFIGS
    if CONFIGS[cfg].get("kind") != "mlp":
        return None
    path = traffic_path(cfg)
    if not os.path.exists(path):
        return None
    with open(path) as fh:
        for line in fh:
            if line.startswith("traffic-record: "):
                rec = json.loads(line[len("traffic-record: "):])
                if rec.get("source_sha256") != kernel_source_digest() or \
                        rec.get("config_id") != cfg:
                    return None
                v = rec["per_launch"].get(kernel_name)
                return None if v is None else v["traffic_bytes"]
    return None


def calibrate_copy():
    import torch
    n = 256 << 20
    src = torch.ones(n, dtype=torch.uint8, device="cuda:0")
    dst = torch.empty_like(src)
    for _ in range(3):
        dst.copy_(src)
    torch.cuda.synchronize()
    print(json.dumps({"copy_bytes": n, "copies": 3}), flush=True)


def linear_flops(T, k, n, r):
    """fwd 2Tkn + 2Tr(k+n) plus bwd 2Tnk + 4Tr(n+k) of one LoRA linear (with dX)."""
    return 4 * T * k * n + 6 * T * r * (k + n)


def mlp_flops(T, d, f, r):
    # fwd: 3 x (2 T k n + 2 T r (k + n)); bwd: 3 x (2 T n k + 4 T r (n + k))
    return 12 * T * d * f + 18 * T * r * (d + f)


def mlp_phase_flops(T, d, f, r):
    """Algorithmic FLOPs of the MLP forward and of its backward."""
    return 6 * T * d * f + 6 * T * r * (d + f), 6 * T * d * f + 12 * T * r * (d + f)


def gemm_flops(kc, T, d, f, r):
    """Algorithmic FLOPs of one launch of each timed GEMM class."""
    import lora_linear_fwd_amd as L
    if kc == L.KC_GATEUP_FWD:     # two LoRA linears d -> f
        return 2 * (2 * T * d * f + 2 * T * r * (d + f))
    if kc == L.KC_DOWN_FWD:       # one LoRA linear f -> d
        return 2 * T * f * d + 2 * T * r * (d + f)
    if kc == L.KC_DOWN_BWD:       # dh = dY Wd + s (dY Bd) Ad
        return 2 * T * d * f + 2 * T * r * (d + f)
    if kc == L.KC_GATEUP_BWD:     # dX = de Wg + dg Wu + LoRA terms
        return 2 * (2 * T * f * d + 2 * T * r * (d + f))
    raise ValueError(kc)


def cpu_baseline(cfg, tokens, mi, reps=2):
    """The float64 CPU oracle on the first `tokens` tokens of the same
    workload (same weights): one warm-up on 512 tokens, then `reps` timed
    forward+backward passes."""
    import numpy as np
    import oracle
    from lora_inputs import CONFIGS
    c = CONFIGS[cfg]
    tokens = min(tokens, c["T"])
    W = dict(mi.W)
    if mi.q4:
        W = {p: oracle.decode_q4_weight(q) for p, q in mi.q4.items()}
    s = oracle.scaling(mi.alpha, mi.r)
    X, dY = mi.X[:tokens].astype(np.float64), mi.dY[:tokens].astype(np.float64)
    Wf = {p: np.asarray(v, np.float64) for p, v in W.items()}
    Af = {p: np.asarray(v, np.float64) for p, v in mi.A.items()}
    Bf = {p: np.asarray(v, np.float64) for p, v in mi.B.items()}
    oracle.mlp_bwd(X[:512], Wf, Af, Bf, s, dY[:512])       # warm-up
    tf = tb = 0.0
    for _ in range(reps):
        t0 = time.perf_counter()
        oracle.mlp_fwd(X, Wf, Af, Bf, s)
        t1 = time.perf_counter()
        oracle.mlp_bwd(X, Wf, Af, Bf, s, dY)
        t2 = time.perf_counter()
        tf += t1 - t0
        tb += t2 - t1
    tf, tb = tf / reps, tb / reps
    dt = tf + tb
    fl = mlp_flops(tokens, c["d"], c["f"], c["r"])
    ffl, bfl = mlp_phase_flops(tokens, c["d"], c["f"], c["r"])
    try:
        cores = len(os.sched_getaffinity(0))
    except AttributeError:
        cores = os.cpu_count()
    return {"value": fl / dt / 1e12, "unit": "TFLOP/s", "cores": cores, "kind": "oracle",
            "sample": f"float64 NumPy oracle, MLP fwd+bwd on {tokens} of {c['T']} tokens "
                      f"(d={c['d']}, f={c['f']}, r={c['r']}), mean of {reps} timed reps after "
                      f"a 512-token warm-up, {dt:.2f} s per rep",
            "tokens_per_s": tokens / dt, "seconds_per_rep": dt,
            "fwd_s": round(tf, 3), "bwd_s": round(tb, 3),
            "fwd_tflops": round(ffl / tf / 1e12, 4), "bwd_tflops": round(bfl / tb / 1e12, 4),
            "blas": blas_vendor()}


def blas_vendor():
    """The BLAS library NumPy's matmul runs on, from numpy.show_config."""
    import numpy as np
    try:
        cfg = np.show_config(mode="dicts")
        deps = cfg.get("Build Dependencies", {})
        b = deps.get("blas", {})
        return f"{b.get('name', '?')} {b.get('version', '')}".strip()
    except Exception:   # older NumPy: no dict mode
        return "unknown"


def time_rmsnorm(T, d, reps=20):
    """RMSNorm in front of the MLP (outside the timed step): average kernel
    time of the forward and the backward over `reps` launches each, and the
    HBM rate of their algorithmic bytes (fwd: X, w read, Y, rstd written;
    bwd: X, w, rstd, dY read, dX written)."""
    import torch

    import lora_linear_fwd_amd as L
    from lora_inputs import gen_rmsnorm
    ri = gen_rmsnorm(T, d, "bf16", seed=5)
    up = lambda a: torch.from_numpy(a).to(torch.bfloat16).to("cuda:0")
    X, w, dY = up(ri.X), up(ri.w), up(ri.dY)
    Y = torch.empty_like(X)
    dX = torch.empty_like(X)
    rstd = torch.empty((T,), dtype=torch.float32, device="cuda:0")
    st = torch.cuda.current_stream()
    out = {}
    for name, fn, nbytes in (
            ("fwd", lambda: L.lora_rmsnorm_fwd(X, w, ri.eps, Y=Y, rstd=rstd, stream=st),
             4 * T * d + 2 * d + 4 * T),
            ("bwd", lambda: L.lora_rmsnorm_bwd(X, w, rstd, dY, dX=dX, stream=st),
             6 * T * d + 2 * d + 4 * T)):
        for _ in range(3):
            fn()
        a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        a.record(st)
        for _ in range(reps):
            fn()
        b.record(st)
        torch.cuda.synchronize()
        ms = a.elapsed_time(b) / reps
        out[name + "_ms"] = round(ms, 4)
        out[name + "_GBps"] = round(nbytes / (ms * 1e-3) / 1e9, 1)
    out["T"], out["d"] = T, d
    return out


def _chain_vs_fused(chain, fused, stream, steps):
    """Per-step time of two forms of the same work: blocks of `steps`
    back-to-back steps of each form, alternated three times after one
    untimed block each (so clock or thermal drift affects both); the median
    over the blocks."""
    import numpy as np
    import torch
    ts = {"chain_ms": [], "fused_ms": []}
    for rep in range(4):
        for name, fn in (("chain_ms", chain), ("fused_ms", fused)):
            a, b = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
            a.record(stream)
            for _ in range(steps):
                fn()
            b.record(stream)
            torch.cuda.synchronize()
            if rep:
                ts[name].append(a.elapsed_time(b) / steps)
    res = {k: round(float(np.median(v)), 4) for k, v in ts.items()}
    res["saved_ms"] = round(res["chain_ms"] - res["fused_ms"], 4)
    return res


def time_norm_mlp(L, X, W, A, B, alpha, dY, ws_fwd, ws_bwd, stream, steps=5):
    """RMSNorm + LoRA-SwiGLU MLP, forward + backward, outside the timed
    region: the norm fused into the gate/up projections (folded weights, no
    normalised rows in memory) against the same step as a chain of the
    standalone norm kernels and the MLP calls.  X stands for the raw rows."""
    import numpy as np
    import torch
    T, d = X.shape
    g = np.random.default_rng(6)
    w = torch.from_numpy((1.0 + 0.1 * g.standard_normal(d)).astype(np.float32)).to(
        torch.bfloat16).to(X.device)
    Wf = dict(W, gate=L.lora_fold_norm_weight(W["gate"], w), up=L.lora_fold_norm_weight(W["up"], w))
    f = W["gate"].shape[0]
    r = A["gate"].shape[0]
    Xn = torch.empty_like(X)
    rstd = torch.empty((T,), dtype=torch.float32, device=X.device)
    e = torch.empty((T, f), dtype=X.dtype, device=X.device)
    g_ = torch.empty_like(e)
    Y = torch.empty_like(X)
    dX = torch.empty_like(X)
    out = {"dX": torch.empty_like(X)}
    nf = L.workspace_bytes(L.OP_RMSNORM_MLP_FWD, L.LORA_BF16, 0, T, d, f, r)
    nb = L.workspace_bytes(L.OP_RMSNORM_MLP_BWD, L.LORA_BF16, 0, T, d, f, r)
    ws = torch.empty(max(nf, nb), dtype=torch.uint8, device=X.device)

    def chain():
        L.lora_rmsnorm_fwd(X, w, 1e-5, Y=Xn, rstd=rstd, stream=stream)
        L.lora_swiglu_mlp_fwd(Xn, W, A, B, alpha, Y=Y, e=e, g=g_, workspace=ws_fwd, stream=stream)
        L.lora_swiglu_mlp_bwd(Xn, W, A, B, alpha, e, g_, dY, out=out, workspace=ws_bwd,
                              stream=stream)
        L.lora_rmsnorm_bwd(X, w, rstd, out["dX"], dX=dX, stream=stream)

    def fused():
        L.lora_rmsnorm_swiglu_mlp_fwd(X, w, 1e-5, Wf, A, B, alpha, Y=Y, e=e, g=g_, rstd=rstd,
                                      workspace=ws[:nf], stream=stream)
        L.lora_rmsnorm_swiglu_mlp_bwd(X, w, rstd, Wf, A, B, alpha, e, g_, dY,
                                      out=dict(out, dX=dX), workspace=ws[:nb], stream=stream)

    res = _chain_vs_fused(chain, fused, stream, steps)
    res["source"] = (f"HIP events around blocks of {steps} back-to-back steps of each form, "
                     "alternated three times after an untimed block each, median per-step time, "
                     "after the timed region; chain = lora_rmsnorm_fwd + MLP fwd + MLP bwd + "
                     "lora_rmsnorm_bwd, fused = lora_rmsnorm_swiglu_mlp_fwd + _bwd on norm-folded "
                     "gate/up weights")
    return res


def time_norm_qkv(L, X, W, A, B, alpha, dY, stream, steps=5):
    """RMSNorm + fused q/k/v LoRA projections, forward + backward, outside
    the timed region: the norm folded into the projections (no normalised
    rows in memory) against the chain of the standalone norm kernels and the
    q/k/v calls.  X stands for the raw rows."""
    import numpy as np
    import torch
    T, k = X.shape
    g = np.random.default_rng(7)
    w = torch.from_numpy((1.0 + 0.1 * g.standard_normal(k)).astype(np.float32)).to(
        torch.bfloat16).to(X.device)
    Wf = {p: L.lora_fold_norm_weight(W[p], w) for p in "qkv"}
    Xn = torch.empty_like(X)
    rstd = torch.empty((T,), dtype=torch.float32, device=X.device)
    dX = torch.empty_like(X)
    outs = {p: torch.empty((T, W[p].shape[0]), dtype=X.dtype, device=X.device) for p in "qkv"}
    grads = {"dX": torch.empty_like(X)}

    def chain():
        L.lora_rmsnorm_fwd(X, w, 1e-5, Y=Xn, rstd=rstd, stream=stream)
        L.lora_qkv_fwd(Xn, W, A, B, alpha, out=outs, stream=stream)
        L.lora_qkv_bwd(Xn, W, A, B, alpha, dY, out=grads, stream=stream)
        L.lora_rmsnorm_bwd(X, w, rstd, grads["dX"], dX=dX, stream=stream)

    def fused():
        L.lora_rmsnorm_qkv_fwd(X, w, 1e-5, Wf, A, B, alpha, out=outs, rstd=rstd, stream=stream)
        L.lora_rmsnorm_qkv_bwd(X, w, rstd, Wf, A, B, alpha, dY, out=dict(grads, dX=dX),
                               stream=stream)

    res = _chain_vs_fused(chain, fused, stream, steps)
    res["source"] = (f"HIP events around blocks of {steps} back-to-back steps of each form, "
                     "alternated three times after an untimed block each, median per-step time, "
                     "after the timed region; chain = lora_rmsnorm_fwd + lora_qkv_fwd + "
                     "lora_qkv_bwd + lora_rmsnorm_bwd, fused = lora_rmsnorm_qkv_fwd + _bwd on "
                     "norm-folded q/k/v weights")
    return res


def bench_attn_mlp(args):
    """Config 4: q, k, v (shared input, dX summed) and o LoRA projections plus
    the LoRA-SwiGLU MLP, forward + backward, T = 16384, r = 64."""
    import numpy as np
    import torch

    import lora_linear_fwd_amd as L
    from lora_inputs import CONFIGS, gen_config

    c = CONFIGS[4]
    T, d, dkv, f, r, alpha = c["T"], c["d"], c["d_kv"], c["f"], c["r"], c["alpha"]
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    inp = gen_config(4)
    up = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    att, mi = inp["attn"], inp["mlp"]
    Xa, Xo = up(att["q"].X), up(att["o"].X)
    Wa = {p: up(att[p].W) for p in att}
    Aa = {p: up(att[p].A) for p in att}
    Ba = {p: up(att[p].B) for p in att}
    dYa = {p: up(att[p].dY) for p in att}
    Wm = {p: up(mi.W[p]) for p in mi.W}
    Am = {p: up(mi.A[p]) for p in mi.A}
    Bm = {p: up(mi.B[p]) for p in mi.B}
    Xm, dYm = up(mi.X), up(mi.dY)
    del inp, att, mi
    # frozen dense weights keep a transposed copy made once (as for the MLP
    # workload), so the backward dX GEMMs run over W^T (the fused q/k/v
    # backward reads the three as the K sources of one GEMM)
    keep_wt = not args.weights_as_stored
    Wqkv = {p: Wa[p] for p in ("q", "k", "v")}   # as stored, for the folded-norm timing
    if keep_wt:
        Wm = {p: L.with_transpose(v) for p, v in Wm.items()}
        for p in ("o", "q", "k", "v"):
            Wa[p] = L.with_transpose(Wa[p])
    stream = torch.cuda.current_stream()
    qkv = ("q", "k", "v")

    def step():
        if args.qkv_separate:
            for p in qkv:
                L.lora_linear_fwd(Xa, Wa[p], Aa[p], Ba[p], alpha, stream=stream)
        else:
            L.lora_qkv_fwd(Xa, {p: Wa[p] for p in qkv}, Aa, Ba, alpha, stream=stream)
        L.lora_linear_fwd(Xo, Wa["o"], Aa["o"], Ba["o"], alpha, stream=stream)
        if args.qkv_separate:
            dX = None
            for i, p in enumerate(qkv):
                dX, _, _ = L.lora_linear_bwd(Xa, Wa[p], Aa[p], Ba[p], alpha, dYa[p], dX=dX,
                                             accumulate_dx=i > 0, stream=stream)
        else:
            L.lora_qkv_bwd(Xa, {p: Wa[p] for p in qkv}, Aa, Ba, alpha, dYa, stream=stream)
        L.lora_linear_bwd(Xo, Wa["o"], Aa["o"], Ba["o"], alpha, dYa["o"], stream=stream)
        Y, e, g = L.lora_swiglu_mlp_fwd(Xm, Wm, Am, Bm, alpha, stream=stream)
        L.lora_swiglu_mlp_bwd(Xm, Wm, Am, Bm, alpha, e, g, dYm, stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    t0, t1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    wall0 = time.perf_counter()
    t0.record(stream)
    for _ in range(args.steps):
        step()
    t1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - wall0
    ms = t0.elapsed_time(t1) / args.steps
    flops = (linear_flops(T, d, d, r) * 2 + linear_flops(T, d, dkv, r) * 2
             + mlp_flops(T, d, f, r))
    tflops = flops / (ms * 1e-3) / 1e12
    line = {
        "metric": "LoRA attention projections + SwiGLU MLP fwd+bwd TFLOP/s",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms, 4),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "higher_is_better": True, "scaling": "weak", "vs_baseline": None, "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"q/k/v/o LoRA projections (d={d}, d_kv={dkv}, q/k/v "
                               f"{'separate' if args.qkv_separate else 'fused'}) + LoRA-SwiGLU "
                               f"MLP (f={f}), T={T}, r={r}, alpha={alpha:g}, bf16",
                   "config_id": 4, "T": T, "d": d, "d_kv": dkv, "f": f, "r": r,
                   "base_weights": ("W and a caller-kept W^T (backward dX GEMMs read W^T)"
                                    if keep_wt else "as stored")},
        "wall_s_timed": round(wall, 3), "flops_per_step": flops,
        "roofline": None, "cpu_baseline": None,
    }
    # the RMSNorm in front of q/k/v, fused into them against the chain (not part of value)
    line["rmsnorm_qkv_step"] = time_norm_qkv(L, Xa, Wqkv, Aa, Ba, alpha,
                                             {p: dYa[p] for p in qkv}, stream)
    print(json.dumps(line), flush=True)


def main():
    args = parse()
    if args.gpus != 1:
        print("bench.py measures one GPU only: this build has no multi-GPU path "
              "(run with --gpus 1)", file=sys.stderr)
        sys.exit(2)
    if args.calibrate_copy:
        calibrate_copy()
        return
    if args.summarize_counters:
        print(summarize_counters(*args.summarize_counters, args.config, trace=args.with_trace),
              end="")
        return
    if args.summarize_sq:
        print(summarize_sq(*args.summarize_sq), end="")
        return
    if args.summarize_trace:
        print(summarize_trace(args.summarize_trace[0], int(args.summarize_trace[1])), end="")
        return
    if args.config == 4:
        bench_attn_mlp(args)
        return
    import numpy as np
    import torch

    import lora_linear_fwd_amd as L
    from lora_inputs import CONFIGS, gen_config

    # the same kernels as liblora.so, plus the hook that records HIP events
    # around one GEMM class's launches (include/liblora_timing.h)
    L.use_timing_build()
    c = CONFIGS[args.config]
    T, d, f, r, alpha = c["T"], c["d"], c["f"], c["r"], c["alpha"]
    q4 = c.get("q4", False)
    if args.dq and not q4:
        print("--dq needs a 4-bit workload (--config 5)", file=sys.stderr)
        sys.exit(2)
    wfmt = (2 if args.dq else 1) if q4 else 0
    dev = torch.device("cuda:0")
    torch.cuda.set_device(dev)
    mi = gen_config(args.config, q4=("dq" if args.dq else None))
    up = lambda a: torch.from_numpy(a).to(torch.bfloat16).to(dev)
    if q4:
        W = {p: L.to_device_q4(mi.q4[p]) for p in mi.q4}
    else:
        W = {p: up(mi.W[p]) for p in mi.W}
    W_stored = W
    # frozen dense weights: a transposed copy is made once, at setup, like the
    # weights themselves; the backward dX GEMMs then read W^T K-contiguously
    keep_wt = not q4 and not args.weights_as_stored
    if keep_wt:
        W = {p: L.with_transpose(v) for p, v in W.items()}
    A = {p: up(mi.A[p]) for p in mi.A}
    B = {p: up(mi.B[p]) for p in mi.B}
    X, dY = up(mi.X), up(mi.dY)
    Y = torch.empty((T, d), dtype=torch.bfloat16, device=dev)
    e = torch.empty((T, f), dtype=torch.bfloat16, device=dev)
    g = torch.empty((T, f), dtype=torch.bfloat16, device=dev)
    out = {"dX": torch.empty((T, d), dtype=torch.bfloat16, device=dev)}
    for p in ("gate", "up", "down"):
        out["dA_" + p] = torch.empty_like(A[p])
        out["dB_" + p] = torch.empty_like(B[p])
    # one buffer; each call gets a view of exactly its strategy's size (the
    # library picks the strategy from the size it is handed)
    mflag = L.LORA_WS_MINIMAL if args.minimal_ws else 0
    fwd_bytes = L.workspace_bytes(L.OP_MLP_FWD | mflag, L.LORA_BF16, wfmt, T, d, f, r)
    bwd_bytes = L.workspace_bytes(L.OP_MLP_BWD | mflag, L.LORA_BF16, wfmt, T, d, f, r)
    ws_all = torch.empty(max(fwd_bytes, bwd_bytes), dtype=torch.uint8, device=dev)
    ws_fwd, ws_bwd = ws_all[:fwd_bytes], ws_all[:bwd_bytes]
    stream = torch.cuda.current_stream()

    def step():
        L.lora_swiglu_mlp_fwd(X, W, A, B, alpha, Y=Y, e=e, g=g, workspace=ws_fwd, stream=stream)
        L.lora_swiglu_mlp_bwd(X, W, A, B, alpha, e, g, dY, out=out, workspace=ws_bwd,
                              stream=stream)

    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()

    kcs = [L.KC_GATEUP_FWD, L.KC_DOWN_FWD, L.KC_DOWN_BWD, L.KC_GATEUP_BWD]

    def timed_steps(n, classes):
        """n steps with HIP events around every launch of the given GEMM
        classes (recorded by the library on its launch stream)."""
        ev = {kc: [(torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True))
                   for _ in range(n)] for kc in classes}
        for kc in classes:
            for a_, b_ in ev[kc]:
                a_.record(stream); b_.record(stream)
        torch.cuda.synchronize()
        t_start = torch.cuda.Event(enable_timing=True)
        t_stop = torch.cuda.Event(enable_timing=True)
        w0 = time.perf_counter()
        t_start.record(stream)
        for i in range(n):
            for kc in classes:
                L.time_next(kc, *ev[kc][i])
            step()
        t_stop.record(stream)
        torch.cuda.synchronize()
        w = time.perf_counter() - w0
        per = {kc: float(np.mean([a_.elapsed_time(b_) for a_, b_ in ev[kc]])) for kc in classes}
        return t_start.elapsed_time(t_stop) / n, w, per

    # the dominant GEMM class, from two untimed steps; the timed region then
    # records events around that class only (each event pair adds a few
    # microseconds of launch gap to the step)
    _, _, probe = timed_steps(2, kcs)
    dom = max(kcs, key=lambda kc: probe[kc])
    ms, wall, live = timed_steps(args.steps, [dom])
    # every GEMM class, in a separate pass after the timed region (reported
    # as kernels_ms; not part of value)
    _, _, kms = timed_steps(min(args.steps, 5), kcs)
    kms[dom] = live[dom]

    # with dense weights, the same step reading W as stored (no transposed
    # copy), in a pass after the timed region
    alt = None
    if keep_wt:
        def step_stored():
            L.lora_swiglu_mlp_fwd(X, W_stored, A, B, alpha, Y=Y, e=e, g=g, workspace=ws_fwd,
                                  stream=stream)
            L.lora_swiglu_mlp_bwd(X, W_stored, A, B, alpha, e, g, dY, out=out, workspace=ws_bwd,
                                  stream=stream)
        step_stored()
        a_, b_ = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
        nalt = max(3, min(args.steps, 10))
        a_.record(stream)
        for _ in range(nalt):
            step_stored()
        b_.record(stream)
        torch.cuda.synchronize()
        alt = {"ms_per_step": round(a_.elapsed_time(b_) / nalt, 4),
               "source": f"{nalt} steps after the timed region, HIP events around them"}

    # forward and backward separately, in another pass after the timed region:
    # HIP events around each call on the same stream
    nph = max(3, min(args.steps, 10))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(3)] for _ in range(nph)]
    for e0, e1, e2 in evs:
        e0.record(stream)
        L.lora_swiglu_mlp_fwd(X, W, A, B, alpha, Y=Y, e=e, g=g, workspace=ws_fwd, stream=stream)
        e1.record(stream)
        L.lora_swiglu_mlp_bwd(X, W, A, B, alpha, e, g, dY, out=out, workspace=ws_bwd,
                              stream=stream)
        e2.record(stream)
    torch.cuda.synchronize()
    fwd_flops, bwd_flops = mlp_phase_flops(T, d, f, r)
    phase = {}
    for name, fl, pick in (("fwd", fwd_flops, lambda e0, e1, e2: e0.elapsed_time(e1)),
                           ("bwd", bwd_flops, lambda e0, e1, e2: e1.elapsed_time(e2)),
                           ("fwd+bwd", fwd_flops + bwd_flops, lambda e0, e1, e2: e0.elapsed_time(e2))):
        ts = [pick(*x) for x in evs]
        med = float(np.median(ts))
        phase[name] = {"median_ms": round(med, 4), "min_ms": round(float(np.min(ts)), 4),
                       "tflops_at_median": round(fl / (med * 1e-3) / 1e12, 2), "flops": fl}
    names = dict(zip([L.KC_GATEUP_FWD, L.KC_DOWN_FWD, L.KC_DOWN_BWD, L.KC_GATEUP_BWD], KC_NAMES))
    dom_tflops = gemm_flops(dom, T, d, f, r) / (kms[dom] * 1e-3) / 1e12
    flops = mlp_flops(T, d, f, r)
    tflops = flops / (ms * 1e-3) / 1e12

    line = {
        "metric": "LoRA-SwiGLU-MLP fwd+bwd TFLOP/s & tokens/s; % of bf16 MFMA peak",
        "value": round(tflops, 2),
        "unit": "TFLOP/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms, 4),
        "tokens_per_s": round(T / (ms * 1e-3), 1),
        "pct_of_bf16_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "bf16",
        "data": "synthetic",
        "config": {"workload": f"LoRA-SwiGLU MLP fwd+bwd, T={T} (4x2048), d={d}, f={f}, "
                               f"r={r}, alpha={alpha:g}, "
                               f"{('4-bit (double-quantised constants)' if args.dq else '4-bit') if q4 else 'bf16'} "
                               f"base weights, bf16 adapters",
                   "config_id": args.config, "T": T, "d": d, "f": f, "r": r,
                   "workspace": "minimal" if args.minimal_ws else "fast",
                   "weights": ("W with a caller-kept W^T (made once at setup; the backward dX "
                               "GEMMs read W^T)") if keep_wt else "as stored"},
        "wall_s_timed": round(wall, 3),
        "kernels_ms": {names[kc]: round(kms[kc], 4) for kc in kcs},
        "kernels_ms_source": "roofline kernel: HIP events in the timed region; the others: "
                             "a separate pass of up to 5 steps after it",
        "phases_ms": phase,
        "weights_as_stored": alt,
        "phases_ms_source": f"HIP events around each call, {nph} steps after the timed region",
        "roofline": {"bound": "mfma", "kernel": names[dom], "achieved": round(dom_tflops, 2),
                     "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                     "frac": round(dom_tflops / PEAK_BF16_TFLOPS, 4),
                     "traffic": stored_traffic(args.config, names[dom]),
                     "flops_per_launch": gemm_flops(dom, T, d, f, r),
                     "avg_launch_ms": round(kms[dom], 4)},
        "cpu_baseline": None,
    }
    # the RMSNorm in front of the MLP, timed on its own (not part of value)
    line["rmsnorm_before_mlp"] = time_rmsnorm(T, d)
    if not q4:
        line["rmsnorm_mlp_step"] = time_norm_mlp(L, X, W_stored, A, B, alpha, dY, ws_fwd, ws_bwd,
                                                 stream)
    if not args.no_cpu_baseline:
        line["cpu_baseline"] = cpu_baseline(args.config, args.cpu_tokens, mi)
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
