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


def test_summary_scales_by_the_copy_and_reads_back(tmp_path, monkeypatch):
    copy_kib = (256 << 20) / 1024
    # the copy kernel reads as half its bytes fetched and all of them written
    _write_counters(tmp_path / "cf.csv", [("copyBuffer", copy_kib / 2)] * 3)
    _write_counters(tmp_path / "cw.csv", [("copyBuffer", copy_kib)] * 3)
    gem = ["k_lora_gemm_pp<1, false>", "k_lora_gemm_pp<0, false>", "k_lora_gemm_pp<2, true>",
           "k_lora_gemm_pp<0, true>"]
    fetch = [100.0, 200.0, 300.0, 400.0]       # KiB per dispatch, two steps
    write = [10.0, 20.0, 30.0, 40.0]
    _write_counters(tmp_path / "f.csv", [("k_prep", 1.0)] + list(zip(gem, fetch)) * 2)
    _write_counters(tmp_path / "w.csv", [("k_prep", 1.0)] + list(zip(gem, write)) * 2)
    md = bench.summarize_counters(str(tmp_path / "f.csv"), str(tmp_path / "w.csv"),
                                  str(tmp_path / "cf.csv"), str(tmp_path / "cw.csv"), 3)
    rec = json.loads(md.split("traffic-record: ")[1])
    assert rec["fetch_scale"] == 2.0 and rec["write_scale"] == 1.0
    for i, name in enumerate(bench.KC_NAMES[:4]):
        v = rec["per_launch"][name]
        assert v["fetch_bytes"] == round(fetch[i] * 1024 * 2)
        assert v["write_bytes"] == round(write[i] * 1024)
        assert v["traffic_bytes"] == v["fetch_bytes"] + v["write_bytes"]
    # read back through the same path bench.py uses, keyed by the workload's shape
    monkeypatch.setattr(bench, "TRAFFIC_SUMMARY", str(tmp_path / "gemm_{shape}_hbm_traffic.md"))
    (tmp_path / "gemm_T8192_d4096_f14336_r16_hbm_traffic.md").write_text("# header\n\n" + md)
    name = bench.KC_NAMES[3]
    assert bench.stored_traffic(3, name) == rec["per_launch"][name]["traffic_bytes"]
    assert bench.stored_traffic(3, "no such kernel") is None
    assert bench.stored_traffic(1, name) is None            # not an MLP workload
    # a record taken on other HIP sources is ignored
    monkeypatch.setattr(bench, "kernel_source_digest", lambda: "0" * 64)
    assert bench.stored_traffic(3, name) is None


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
