"""Host-side logic of bench.py: FLOP accounting, the counter summary and the
guarded read-back of the stored traffic record (no GPU needed)."""
import csv
import json
import os

import pytest

import bench


def _lin_fwd(T, k, n, r):
    # X W^T (T x k x n), X A^T (T x k x r), H B^T (T x r x n): 2 flops per multiply-add
    return 2 * T * k * n + 2 * T * k * r + 2 * T * r * n


def _lin_bwd(T, k, n, r):
    # dX = dY W (T x n x k), G = dY B (T x n x r), G A (T x r x k),
    # dA = G^T X (r x T x k), dB = dY^T H (n x T x r); H is kept from the forward
    return 2 * T * n * k + 2 * T * n * r + 2 * T * r * k + 2 * r * T * k + 2 * n * T * r


@pytest.mark.parametrize("T,d,f,r", [(8192, 4096, 14336, 16), (8192, 2048, 8192, 16), (7, 5, 11, 3)])
def test_mlp_flops_are_the_sum_of_the_products(T, d, f, r):
    layers = [(d, f), (d, f), (f, d)]          # gate, up: d -> f; down: f -> d
    fwd = sum(_lin_fwd(T, k, n, r) for k, n in layers)
    bwd = sum(_lin_bwd(T, k, n, r) for k, n in layers)
    assert bench.mlp_phase_flops(T, d, f, r) == (fwd, bwd)
    assert bench.mlp_flops(T, d, f, r) == fwd + bwd
    assert bench.linear_flops(T, d, f, r) == _lin_fwd(T, d, f, r) + _lin_bwd(T, d, f, r)


def test_config3_step_flops():
    assert bench.mlp_flops(8192, 4096, 14336, 16) == 5815922589696


def test_gemm_class_flops_cover_the_dense_work():
    import lora_linear_fwd_amd as L
    T, d, f, r = 8192, 4096, 14336, 16
    kcs = [L.KC_GATEUP_FWD, L.KC_DOWN_FWD, L.KC_DOWN_BWD, L.KC_GATEUP_BWD]
    dense = sum(bench.gemm_flops(kc, T, d, f, r) for kc in kcs) - 12 * T * r * (d + f)
    assert dense == 12 * T * d * f


def _write_counters(path, rows):
    with open(path, "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Value"])
        for i, (name, v) in enumerate(rows):
            w.writerow([i + 1, name, v])


GEMS = ["k_lora_gemm_pp<1, false>", "k_lora_gemm_pp<0, false>", "k_lora_gemm_pp<3, false>",
        "k_lora_gemm_pp<0, false>"]


def _step(values, q4=False, prep=False):
    """One MLP step's dispatches in launch order, the GEMMs carrying `values`.
    prep: the forward makes operand copies first (padded ranks, folded norm);
    at r = 16 it reads the adapters in place and opens with the pass over X."""
    pre = [("k_dequant4(unsigned char const*)", 0.5)] * 2 if q4 else []
    pre += [("k_prep(PrepBatch)", 1.0)] if prep else []
    fwd = pre + [("k_skinny_nt<32, false, 64>(SkinnyNTArgs)", 2.0),
                 ("k_reduce_side", 0.1), (GEMS[0], values[0]), ("k_reduce_dual_u", 0.1),
                 (GEMS[1], values[1])]
    bwd = [("k_prep(PrepBatch)", 1.0), ("k_skinny_nt<16, false, 64>(SkinnyNTArgs)", 2.0),
           ("k_reduce_side", 0.1), ("k_skinny_nt<32, false, 64>(SkinnyNTArgs)", 2.0),
           ("k_reduce_side", 0.1), (GEMS[2], values[2]), ("k_reduce_batch", 0.2),
           (GEMS[3], values[3]), ("k_reduce_tn", 0.3)]
    return fwd + bwd


def test_summary_scales_by_the_copy_and_reads_back(tmp_path, monkeypatch):
    copy_kib = (256 << 20) / 1024
    # the copy kernel reads as half its bytes fetched and all of them written
    _write_counters(tmp_path / "cf.csv", [("copyBuffer", copy_kib / 2)] * 3)
    _write_counters(tmp_path / "cw.csv", [("copyBuffer", copy_kib)] * 3)
    fetch = [100.0, 200.0, 300.0, 400.0]       # KiB per dispatch
    write = [10.0, 20.0, 30.0, 40.0]
    # steps 2-5 carry the values; the warm-up step and a later pass of other
    # forms (here 9x) must not enter the averages
    f_rows = _step([9 * v for v in fetch]) + sum((_step(fetch) for _ in range(4)), []) \
        + _step([9 * v for v in fetch])
    w_rows = _step([9 * v for v in write]) + sum((_step(write) for _ in range(4)), []) \
        + _step([9 * v for v in write])
    _write_counters(tmp_path / "f.csv", f_rows)
    _write_counters(tmp_path / "w.csv", w_rows)
    md = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                  str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 3)
    rec = json.loads(md.split("traffic-record: ")[1])
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0 and rec["config_id"] == 3
    for i, name in enumerate(bench.KC_NAMES[:4]):
        v = rec["per_launch"][name]
        assert v["fetch_bytes"] == round(fetch[i] * 1024 * 2)
        assert v["write_bytes"] == round(write[i] * 1024)
        assert v["traffic_bytes"] == v["fetch_bytes"] + v["write_bytes"]
    # the per-dispatch table lists step 2, every dispatch of it
    assert md.count("| `") == len(_step(fetch))
    # read back through the same path bench.py uses, keyed by the workload's shape
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "gemm_{shape}_hbm_traffic.md"))
    assert bench.traffic_path(3).endswith("gemm_T8192_d4096_f14336_r16_hbm_traffic.md")
    assert bench.traffic_path(5).endswith("gemm_T8192_d4096_f14336_r16_q4_hbm_traffic.md")
    (tmp_path / "gemm_T8192_d4096_f14336_r16_hbm_traffic.md").write_text("# header\n\n" + md)
    name = bench.KC_NAMES[3]
    assert bench.stored_traffic(3, name) == rec["per_launch"][name]["traffic_bytes"]
    assert bench.stored_traffic(3, "no such kernel") is None
    assert bench.stored_traffic(1, name) is None            # not an MLP workload
    # the 4-bit workload of the same shape has a record of its own
    (tmp_path / "gemm_T8192_d4096_f14336_r16_q4_hbm_traffic.md").write_text("# header\n\n" + md)
    assert bench.stored_traffic(5, name) is None            # recorded for workload 3
    # a record taken on other HIP sources is ignored
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.stored_traffic(3, name) is None


@pytest.mark.parametrize("prep", [False, True], ids=["in-place", "prep"])
def test_steps_start_at_the_forward_and_its_4bit_decodes(prep):
    rows = [(i, n, 0.0) for i, (n, _) in enumerate(
        [("k_reduce_tn", 0)] + _step([1] * 4, q4=True, prep=prep)
        + _step([1] * 4, q4=True, prep=prep))]
    steps = bench._steps(rows)
    assert len(steps) == 2
    for st in steps:
        assert "k_dequant4(" in st[0][1] and "k_dequant4(" in st[1][1]
        assert ("k_prep" in st[2][1]) == prep
        assert len(st) == len(_step([1] * 4, q4=True, prep=prep))


@pytest.mark.parametrize("prep", [False, True], ids=["in-place", "prep"])
def test_steps_of_a_dense_mlp_skip_the_backward_pass_over_x(prep):
    """The backward's 32-wide pass over X follows a reduction: no step opens
    there, with or without the forward's operand copies."""
    seq = sum((_step([1] * 4, prep=prep) for _ in range(3)), [])
    starts = bench._step_starts([n for n, _ in seq])
    assert starts == [i * len(_step([1] * 4, prep=prep)) for i in range(3)]


def test_steps_of_the_attention_workload_open_at_the_fused_qkv():
    """q/k/v forward (k_prep, then the rank-3r pass over X), o, MLP: one step
    per q/k/v opener; the MLP's own k_prep inside the step opens nothing."""
    one = ["k_prep", "k_skinny_nt<192, false, 128>", "k_reduce_side", "k_lora_gemm_pp<0, false>",
           "k_prep", "k_skinny_nt<64, false, 128>", "k_reduce_side", "k_lora_gemm_pp<0, false>",
           "k_prep", "k_skinny_nt<128, false, 128>", "k_reduce_side", "k_lora_gemm_pp<1, false>",
           "k_reduce_tn"]
    rows = [(i, n, 0.0) for i, n in enumerate(one * 3)]
    steps = bench._steps(rows)
    assert [len(st) for st in steps] == [len(one)] * 3


def test_sq_summary_medians_per_class(tmp_path):
    """Clock, TFLOP/s and MFMA-busy fraction from two counter sets."""
    dur_ns = 1_000_000                                   # 1 ms per GEMM dispatch
    clk = 1.5e9
    sets = {1: {"SQ_INSTS_VALU_MFMA_MOPS_BF16": 2.0e12 / 512 * 1e-3 * 1e3,
                "SQ_VALU_MFMA_BUSY_CYCLES": 0.8 * 1024 * clk * 1e-3,
                "SQ_LDS_BANK_CONFLICT": 7.0, "SQ_WAIT_INST_LDS": 1.0, "SQ_WAVE_CYCLES": 10.0},
            2: {"GRBM_GUI_ACTIVE": 8 * clk * 1e-3}}
    for k, counters in sets.items():
        with open(tmp_path / f"sq{k}.csv", "w", newline="") as fh:
            w = csv.writer(fh)
            w.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                        "Start_Timestamp", "End_Timestamp"])
            t = 0
            for i, (n, _) in enumerate(sum((_step([0] * 4) for _ in range(6)), [])):
                for cn, cv in counters.items():
                    w.writerow([i + 1, n, cn, cv, t, t + dur_ns])
                t += dur_ns
    md = bench.summarize_sq(str(tmp_path / "sq1.csv"), str(tmp_path / "sq2.csv"))
    rows = [l for l in md.splitlines() if l.startswith("| ") and "| dispatches |" not in l]
    assert len(rows) == 4
    for l in rows:
        c = [x.strip() for x in l.strip("|").split("|")]
        assert c[1] == "4" and c[2] == "1.000" and c[3] == "1.50"
        assert c[4] == "2000" and c[6] == "80 %" and c[7] == "7" and c[8] == "10.0 %"


def test_trace_summary_lists_one_step(tmp_path):
    with open(tmp_path / "run_kernel_stats.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs",
                    "MaxNs"])
        w.writerow([GEMS[0], 3, 3000, 1000, 50.0, 900, 1100])
    with open(tmp_path / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        t = 0
        for n, _ in sum((_step([0] * 4) for _ in range(3)), []):
            w.writerow([n, t, t + 2000])
            t += 3000                                    # 1 us gap before each dispatch
    md = bench.summarize_trace(str(tmp_path), 1)
    assert "| `k_lora_gemm_pp<1, false>` | 3 | 1.0 | 0.9 | 1.1 | 50.00 |" in md
    assert "Step 2 of 3" in md
    lines = [l for l in md.splitlines() if " dur " in l]
    assert len(lines) == len(_step([0] * 4))
    assert lines[0].split()[0] == "0.0" and lines[1].split()[2] == "1.0"


def test_source_digest_covers_every_hip_source(tmp_path, monkeypatch):
    for n in ("a.hip", "b.hpp"):
        (tmp_path / n).write_text("x")
    monkeypatch.setattr(bench, "CSRC", str(tmp_path))
    d0 = bench.kernel_source_digest()
    (tmp_path / "b.hpp").write_text("y")
    assert bench.kernel_source_digest() != d0
    (tmp_path / "b.hpp").write_text("x")
    assert bench.kernel_source_digest() == d0
    os.remove(tmp_path / "a.hip")
    assert bench.kernel_source_digest() != d0


def test_counter_summary_pairs_dispatches_with_traced_durations(tmp_path):
    copy_kib = (256 << 20) / 1024
    _write_counters(tmp_path / "cf.csv", [("copyBuffer", copy_kib / 2)] * 3)
    _write_counters(tmp_path / "cw.csv", [("copyBuffer", copy_kib)] * 3)
    loop = [("k_rmsnorm_fwd<false>", 1000.0)] * 12
    rows = sum((_step([100.0] * 4) for _ in range(6)), []) + loop
    _write_counters(tmp_path / "f.csv", rows)
    _write_counters(tmp_path / "w.csv", rows)
    # a trace of the same dispatches, 2 us each
    with open(tmp_path / "run_kernel_trace.csv", "w", newline="") as fh:
        w = csv.writer(fh)
        w.writerow(["Kernel_Name", "Start_Timestamp", "End_Timestamp"])
        for i, (n, _) in enumerate(rows):
            w.writerow([n, 3000 * i, 3000 * i + 2000])
    md = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                  str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 3,
                                  trace=(str(tmp_path), "3"))
    # GEMM 3 of the step: 100 KiB fetched (x2 by the copy scale) + 100 KiB written in 2 us
    gb = (100 * 1024 * 2 + 100 * 1024) / 2e-6 / 1e9
    assert f"| 2.0 | {gb:.0f} | {gb / 8000:.2f} |" in md
    # the norm loop: 12 dispatches, 1000 KiB x 3 per 2 us
    gl = 3000 * 1024 / 2e-6 / 1e9
    assert f"| `k_rmsnorm_fwd<false>` | 12 | 2.0 | 1.0 | 2.0 | {gl:.0f} |" in md
