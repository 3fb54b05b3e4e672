"""Host-side tools of bench.py: the kernel-source hash that keys the traffic
summaries, and the counter scaling that turns FETCH_SIZE / WRITE_SIZE into
bytes (CPU only)."""
import csv
import json
import os

import pytest

import bench

KIB = 1024


def test_code_hash_ignores_comments_and_layout():
    a = "int f(int x) {\n    return x + 1;  // one more\n}\n"
    b = "/* the successor */\nint f(int x)\n{\n  return x + 1;\n}\n"
    c = "int f(int x) {\n    return x + 2;  // one more\n}\n"
    assert bench._code_only(a) == bench._code_only(b)
    assert bench._code_only(a) != bench._code_only(c)


def test_kernel_source_hash_covers_each_source_set():
    h_dec = bench.kernel_source_hash("b1_topk2048_n32768_paged_bf16")
    h_idx = bench.kernel_source_hash("idx_b16_topk2048_n65536")
    assert len(h_dec) == 16 and len(h_idx) == 16 and h_dec != h_idx
    assert bench.kernel_source_hash("b64_topk2048_n1k-128k_paged_bf16") == h_dec


def _write_counters(path, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for i, (kernel, counter, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i, "Kernel_Name": kernel, "Counter_Name": counter, "Counter_Value": value})


def test_traffic_scale_uses_only_the_probe_dispatches(tmp_path, monkeypatch):
    # The probe's input comes from a fill kernel that reads nothing.  Averaging
    # it in with the three bitwise_not dispatches would put the fetch scale at
    # 8/3 instead of 2 and overstate every fetch by 4/3.
    fill = "void at::native::vectorized_elementwise_kernel<16, at::native::FillFunctor<unsigned char>>"
    bnot = "void at::native::vectorized_elementwise_kernel<16, at::native::bitwise_not_kernel_cuda>"
    probe = bench.COPY_PROBE_BYTES
    _write_counters(tmp_path / "cf", [(fill, "FETCH_SIZE", 26)] + [(bnot, "FETCH_SIZE", probe / 2 / KIB)] * 3)
    _write_counters(tmp_path / "cw", [(fill, "WRITE_SIZE", probe / KIB)] + [(bnot, "WRITE_SIZE", probe / KIB)] * 3)
    part = "smla::(anonymous namespace)::partial_kernel<0>(smla::(anonymous namespace)::PartialArgs)"
    comb = "smla::(anonymous namespace)::combine_kernel<4>(...)"
    _write_counters(tmp_path / "f", [(part, "FETCH_SIZE", 1000.0), (comb, "FETCH_SIZE", 5000.0),
                                     (part, "FETCH_SIZE", 1100.0)])
    _write_counters(tmp_path / "w", [(part, "WRITE_SIZE", 2048.0), (comb, "WRITE_SIZE", 64.0)])
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    monkeypatch.setattr(bench, "kernel_source_hash", lambda workload: "0123456789abcdef")
    assert bench.traffic_summary("b1_topk2048_n32768_paged_bf16", str(tmp_path / "f"), str(tmp_path / "w"),
                                 str(tmp_path / "cf"), str(tmp_path / "cw"), command="test") == 0
    rec = json.load(open(tmp_path / "profiles" / "traffic_b1_topk2048_n32768_paged_bf16.json"))
    assert rec["copy_probe"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["copy_probe"]["write_scale"] == pytest.approx(1.0)
    # only the partial kernel's dispatches: mean 1050 KiB fetched, 2048 KiB written
    assert rec["fetch_bytes_per_launch"] == round(1050 * KIB * 2.0)
    assert rec["write_bytes_per_launch"] == 2048 * KIB
    assert rec["dispatches"] == {"fetch": 2, "write": 1}
    assert rec["kernel_source_hash"] == "0123456789abcdef"
