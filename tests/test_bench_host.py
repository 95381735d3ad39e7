"""Host logic of bench.py (no GPU): the algorithmic work a benchmark line is
priced on, the kernel a workload's attention launch runs, and the traffic
record (counter parsing, copy-probe scaling, the source-hash guard)."""

import csv
import json
import os

import pytest

import bench
import datagen


def test_algorithmic_work_of_the_metric_workload():
    sh = datagen.WORKLOADS["dream_gqa"]
    a = bench.algorithmic(sh)
    # B4, Hq28 over Hkv4, d128, P32768 + Bq32 keys: QK^T + PV = 4 flops per
    # (query row, key, head dim); K/V bf16 read once per kv-head, Q read once
    n_keys = 32768 + 32
    assert a["flops"] == 4 * 4 * 28 * 32 * n_keys * 128 == 60_188_262_400
    kv = 2 * 4 * 4 * n_keys * 128 * 2
    q = 4 * 28 * 32 * 128 * 2
    assert a["kernel_bytes"] == kv + q == 269_615_104
    assert a["units"] == 16 and a["unit_bytes"] * 16 == pytest.approx(kv + q)
    # prefix only (the prefix partial): the block's keys drop out
    p = bench.algorithmic(sh, with_block=False)
    assert p["flops"] == 4 * 4 * 28 * 32 * 32768 * 128


def test_algorithmic_work_counts_retained_rows_and_their_indices():
    sh = datagen.WORKLOADS["sparse_gqa"]
    a = bench.algorithmic(sh)
    n_keys = 8192 + 64   # kept prefix rows + block keys
    assert a["flops"] == 4 * 2 * 28 * 64 * n_keys * 128
    assert a["kernel_bytes"] == 2 * 2 * 4 * n_keys * 128 * 2 + 2 * 28 * 64 * 128 * 2 + 4 * 2 * 4 * 8192


@pytest.mark.parametrize("name,kernel", [
    ("dream_gqa", "attn_bf16_pp_kernel"),     # 7 x 32 = 224 packed rows
    ("sparse_gqa", "attn_bf16_pp_kernel"),    # 7 x 64 = 448 rows: two chunks of 224
    ("llada_bf16", "attn_bf16_kernel"),       # 32 rows: one row wave
    ("reuse_bf16", "attn_bf16_kernel"),
    ("tiny_f32", "attn_f32_kernel"),
])
def test_attention_kernel_name(name, kernel):
    assert bench.attention_kernel_name(datagen.WORKLOADS[name]) == kernel


def _write_counters(path, kernel, values):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Kernel_Name", "Counter_Name", "Counter_Value"])
        w.writeheader()
        w.writerow({"Kernel_Name": "void other_kernel(int)", "Counter_Name": "X", "Counter_Value": 1.0})
        for v in values:
            w.writerow({"Kernel_Name": f"void ns::{kernel}<128, true>(Params)", "Counter_Name": "X",
                        "Counter_Value": v})


def test_record_traffic_scales_by_the_copy_probe(tmp_path):
    top = str(tmp_path / "pmc")
    _write_counters(os.path.join(top, "pmc_fetch"), "attn_bf16_pp_kernel", [100.0, 300.0])   # mean 200 KiB
    _write_counters(os.path.join(top, "pmc_write"), "attn_bf16_pp_kernel", [50.0])
    # the 1 GiB copy counts 524288 KiB fetched (scale 2) and 1048576 KiB written (scale 1)
    _write_counters(os.path.join(top, "pmc_cfetch"), "copyBuffer", [524288.0])
    _write_counters(os.path.join(top, "pmc_cwrite"), "copyBuffer", [1048576.0])
    out = str(tmp_path / "rec.json")
    bench.record_traffic(top, out)
    rec = json.load(open(out))
    assert rec["copy_probe"]["fetch_scale"] == pytest.approx(2.0)
    assert rec["copy_probe"]["write_scale"] == pytest.approx(1.0)
    assert rec["bytes_per_launch"] == 200 * 1024 * 2 + 50 * 1024
    assert rec["kernel_sources_sha256"] == bench.sources_sha256(rec["kernel_sources"])


def test_measured_traffic_is_guarded_by_the_source_hash(tmp_path):
    sh = datagen.WORKLOADS["dream_gqa"]
    rec = {"kernel_sources": list(bench.KERNEL_SOURCES),
           "kernel_sources_sha256": bench.sources_sha256(bench.KERNEL_SOURCES),
           "bytes_per_launch": 123456}
    good = tmp_path / "good.json"
    good.write_text(json.dumps(rec))
    assert bench.measured_traffic(str(good), sh) == 123456
    stale = tmp_path / "stale.json"
    stale.write_text(json.dumps(dict(rec, kernel_sources_sha256="0" * 64)))
    assert bench.measured_traffic(str(stale), sh) is None
    # a record belongs to the metric workload only
    assert bench.measured_traffic(str(good), datagen.WORKLOADS["llada_bf16"]) is None
    assert bench.measured_traffic(str(tmp_path / "missing.json"), sh) is None


def test_committed_traffic_record_matches_the_kernel_sources():
    path = os.path.join(bench.ROOT, "profiles", "attn_bf16_dream_gqa_traffic.json")
    rec = json.load(open(path))
    if rec["kernel_sources_sha256"] != bench.sources_sha256(rec["kernel_sources"]):
        # the benchmark then reports traffic as null, as it should
        pytest.skip("the kernel sources changed since the counters were taken: record them again")
    assert bench.measured_traffic(path, datagen.WORKLOADS["dream_gqa"]) == rec["bytes_per_launch"]
