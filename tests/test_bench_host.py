"""Host logic of bench.py (no GPU): the one-GPU guard, the algorithmic work
figures and the reduction of rocprofv3 counter output to HBM bytes."""
import csv
import os
import sys

import pytest

sys.path.insert(0, os.path.dirname(os.path.dirname(os.path.abspath(__file__))))
import bench  # noqa: E402
import learned_token_pruning_03_amd.workloads as W  # noqa: E402


def test_more_than_one_gpu_is_refused_with_a_message(capsys):
    assert bench.main(["--gpus", "2"]) == 2
    assert "one GPU" in capsys.readouterr().err


def test_attention_flops_count_visible_pairs():
    sh = W.SHAPES["qwen1p7b_32k"]
    # K = 4096 kept queries, causal: K (K + 1) / 2 visible pairs, 2 products of Dh MACs each.
    assert bench.attn_flops(sh) == 4.0 * 128 * 16 * 4096 * 4097 / 2
    by = bench.stage_bytes(sh)
    assert by["select"] == 32768 * 4 + 4096 * 4
    assert by["gather"] == 2 * 4096 * (2048 * 2 + 8)


def _write_counters(folder, rows):
    os.makedirs(folder, exist_ok=True)
    with open(os.path.join(folder, "x_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        for r in rows:
            w.writerow(r)


def test_traffic_summary_scales_each_counter_by_the_copy_kernel(tmp_path):
    true_kib = bench.COPY_CAL_ELEMS * 4 / 1024
    fetch, write = str(tmp_path / "f"), str(tmp_path / "w")
    # FETCH_SIZE reads half the true bytes of the calibration copy; the attention
    # kernel's rows (two per dispatch, summed) give 1000 KiB per dispatch.
    _write_counters(fetch, [
        {"Dispatch_Id": 1, "Kernel_Name": "attn_bf16_pp_kernel<128>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 600},
        {"Dispatch_Id": 1, "Kernel_Name": "attn_bf16_pp_kernel<128>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 400},
        {"Dispatch_Id": 2, "Kernel_Name": "attn_bf16_pp_kernel<128>", "Counter_Name": "FETCH_SIZE", "Counter_Value": 1000},
        {"Dispatch_Id": 3, "Kernel_Name": "neg_kernel", "Counter_Name": "FETCH_SIZE", "Counter_Value": true_kib / 2},
    ])
    _write_counters(write, [
        {"Dispatch_Id": 1, "Kernel_Name": "attn_bf16_pp_kernel<128>", "Counter_Name": "WRITE_SIZE", "Counter_Value": 300},
        {"Dispatch_Id": 3, "Kernel_Name": "neg_kernel", "Counter_Name": "WRITE_SIZE", "Counter_Value": true_kib},
    ])
    rec = bench.traffic_summary(fetch, write)
    assert rec["fetch_calibration"]["scale"] == pytest.approx(2.0)
    assert rec["write_calibration"]["scale"] == pytest.approx(1.0)
    assert rec["fetch_bytes_per_launch"] == 2 * 1000 * 1024
    assert rec["write_bytes_per_launch"] == 300 * 1024
    assert rec["hbm_bytes_per_launch"] == 2 * 1000 * 1024 + 300 * 1024
    assert rec["dispatches"] == {"fetch": 2, "write": 1}


def test_stored_traffic_applies_only_to_its_workload_and_kernel_source():
    # The committed PMC summary was taken on the 32k workload; other
    # workloads get no traffic figure.
    assert bench.load_traffic("qwen1p7b_128k") is None
    assert bench.load_traffic("stack19") is None
    t = bench.load_traffic("qwen1p7b_32k")
    assert t is None or t > 0
