"""The benchmark's host-side logic, without a GPU: the refusal of more than
one GPU, the algorithmic bytes the roofline is priced on, and the traffic
record made from two rocprofv3 counter runs (FETCH_SIZE, WRITE_SIZE) scaled
by a plain copy of known size."""
import csv
import json
import os
import subprocess
import sys
from types import SimpleNamespace

import numpy as np
import pytest

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert res.returncode == 2
    assert "one GPU" in res.stderr
    assert res.stdout == ""


def _decode_shape(lens, next_n=1, mxfp4=False):
    lens = np.asarray(lens, np.int32)
    return SimpleNamespace(
        context_lens=lens, rows=lens.size, mxfp4=mxfp4,
        request_keys=lambda: lens.reshape(-1, next_n).max(axis=1))


def test_long_decode_algorithmic_bytes():
    # B=8 requests of 131072 keys: K 128 B and one fp32 scale per key, one fp32
    # logit per key, 2048 block-table entries per request, Q (32x128 fp8),
    # 32 fp32 weights and the length per row, and the 1024-bin histogram
    # read and written once per row.
    ab = bench.algorithmic_bytes(_decode_shape([131072] * 8))
    assert ab["k"] == 8 * 131072 * 128 == 134_217_728
    assert ab["total"] == 142_771_232


def test_algorithmic_bytes_ragged_and_verify_rows():
    # Two requests with next_n=2: the K sweep reads each request once, up to
    # its longest row; logits are per row; a partial page still costs a
    # whole block-table entry.
    ab = bench.algorithmic_bytes(_decode_shape([100, 65, 0, 3], next_n=2))
    keys = 100 + 3
    assert ab["k"] == keys * 128
    want = keys * 132 + (100 + 65 + 3) * 4 + (2 + 1) * 4 + 4 * (4096 + 128 + 4) + 4 * 8192
    assert ab["total"] == want


def test_algorithmic_bytes_mxfp4_tokens():
    # A packed MXFP4 token is 64 B of codes and 4 E8M0 block scales; no
    # separate fp32 scale.
    ab = bench.algorithmic_bytes(_decode_shape([64] * 2, mxfp4=True))
    assert ab["k"] == 128 * 68
    assert ab["total"] == 128 * 68 + 128 * 4 + 2 * 4 + 2 * (4096 + 128 + 4) + 2 * 8192


def _write_counters(path, counter, rows):
    os.makedirs(path, exist_ok=True)
    with open(os.path.join(path, "run_counter_collection.csv"), "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name",
                                          "Counter_Value"])
        w.writeheader()
        for i, (name, value) in enumerate(rows):
            w.writerow({"Dispatch_Id": i + 1, "Kernel_Name": name, "Counter_Name": counter,
                        "Counter_Value": value})


LOGITS = bench.LOGITS_KERNEL + "(LogitsArgs, int)"
COPY = "void at::native::elementwise_kernel_copy"


def test_traffic_record_scales_by_the_copy(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    # FETCH_SIZE reads the copy's bytes at half (factor 2); a logits launch
    # before the copies is averaged, other kernels and copies before the last
    # logits dispatch are ignored.
    _write_counters(tmp_path / "f", "FETCH_SIZE", [
        (COPY, 1.0), (LOGITS, 1000.0), ("topk_row_kernel", 9e9), (LOGITS, 1200.0),
        (COPY, copy_kib / 2), (COPY, copy_kib / 2)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [
        (LOGITS, 300.0), (LOGITS, 300.0), (COPY, copy_kib)])
    tr = bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"), "long_decode")
    assert tr["workload"] == "long_decode"
    assert tr["kernel_src_sha"] == bench.kernel_source_digest()
    assert tr["FETCH_SIZE"]["dispatches"] == 2 and tr["FETCH_SIZE"]["copies"] == 2
    assert tr["FETCH_SIZE"]["factor"] == pytest.approx(2.0)
    assert tr["FETCH_SIZE"]["bytes_per_launch"] == pytest.approx(1100.0 * 1024 * 2)
    assert tr["WRITE_SIZE"]["factor"] == pytest.approx(1.0)
    assert tr["bytes_per_launch"] == round(1100.0 * 1024 * 2 + 300.0 * 1024)


def test_traffic_record_needs_a_copy_after_the_logits(tmp_path):
    _write_counters(tmp_path / "f", "FETCH_SIZE", [(COPY, 5.0), (LOGITS, 10.0)])
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(LOGITS, 1.0), (COPY, 2.0)])
    with pytest.raises(SystemExit, match="calibration copy"):
        bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"), "long_decode")


def test_committed_traffic_record_is_close_to_the_algorithmic_bytes():
    # The committed counter record of the long-decode launch: HBM bytes within
    # a few percent of the algorithmic minimum (no re-reads), and its kernel
    # digest names a source state (the bench drops the figure when the digest
    # differs from the current source).
    with open(bench.TRAFFIC_FILE) as f:
        tr = json.load(f)
    assert tr["workload"] == "long_decode"
    assert len(tr["kernel_src_sha"]) == 16
    total = bench.algorithmic_bytes(_decode_shape([131072] * 8))["total"]
    assert total <= tr["bytes_per_launch"] <= 1.05 * total


def test_page_list_is_each_requests_live_pages_in_order():
    import gen
    x = gen.make_indexer_inputs("pl", 3, 2, [64, 130, 1], 5)
    got = bench.page_list(x)
    # request b's rows see base + j keys (next_n = 2): 65, 131 and 2 keys ->
    # 2, 3 and 1 pages of its block-table row
    want = np.concatenate([x.block_table[0, :2], x.block_table[1, :3], x.block_table[2, :1]])
    assert got.dtype == np.int32 and np.array_equal(got, want)


def test_sampled_cpu_baseline_scales_by_row_key_pairs():
    import gen
    x = gen.make_indexer_inputs("cb", 4, 1, [3000, 1000, 1000, 1000], 6)
    out = bench.sampled_cpu_baseline(x, budget_rows_keys=4000)
    assert out["kind"] == "oracle" and out["unit"] == "us/step" and out["cores"] >= 1
    assert "2 of 4 requests (4000 of 6000 row-key pairs)" in out["sample"]
    assert out["value"] > 0


def test_gpu_clock_reader_returns_a_mapping():
    assert isinstance(bench.gpu_clock_mhz(), dict)


def test_every_workload_names_its_counted_kernel_and_profile_args():
    import gen
    for w in gen.CONFIG_NAMES + gen.MXFP4_CONFIG_NAMES + gen.PREFILL_CONFIG_NAMES:
        assert w in bench.COUNTED_KERNEL
        args = bench.profile_args(w, 5)
        assert "--no-cpu-baseline" in args and "--sweep-steps 0" in args
        if w.startswith("prefill/"):
            assert "--prefill-steps 5" in args
        else:
            assert f"--workload {w} " in args and "--prefill-steps 0" in args
    assert bench.traffic_file("spec_verify/unit").endswith("logits_spec_verify_unit_traffic.json")


def test_traffic_record_of_another_workload_reads_its_kernel(tmp_path):
    copy_kib = bench.COPY_BYTES / 1024
    pf = "void pmqa::(anonymous namespace)::indexer_prefill_logits_kernel<0>(pmqa::PrefillArgs)"
    # an upload copy after the kernel's last dispatch is not a calibration copy
    _write_counters(tmp_path / "f", "FETCH_SIZE", [
        (LOGITS, 50.0), (pf, 400.0), (pf, 600.0), (COPY, 3.0)] + [(COPY, copy_kib / 2)] * 3)
    _write_counters(tmp_path / "w", "WRITE_SIZE", [(LOGITS, 9.0), (pf, 100.0), (COPY, copy_kib)])
    tr = bench.traffic_from(str(tmp_path / "f"), str(tmp_path / "w"), "prefill/extend")
    assert tr["kernel"] == bench.COUNTED_KERNEL["prefill/extend"]
    assert tr["FETCH_SIZE"]["dispatches"] == 2
    assert tr["bytes_per_launch"] == round(500.0 * 1024 * 2 + 100.0 * 1024)
    md = bench.write_traffic_md(tr, 1_000_000, out_dir=str(tmp_path))
    text = open(md).read()
    assert "--traffic-from" in text and "prefill/extend" in text and "--prefill-steps 5" in text


def test_stats_and_counter_summaries(tmp_path):
    st = tmp_path / "run_kernel_stats.csv"
    with open(st, "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Name", "Calls", "AverageNs", "MinNs", "MaxNs"])
        w.writeheader()
        w.writerow({"Name": "void pmqa::(anonymous namespace)::topk_finish_kernel<0, false>(int)",
                    "Calls": 7, "AverageNs": 8000.0, "MinNs": 7000, "MaxNs": 9000})
    md = open(bench.write_stats_md(str(st), "varlen_decode", 5, out_dir=str(tmp_path))).read()
    assert "| topk_finish_kernel<0, false> | 7 | 8.00 | 7.00 | 9.00 |" in md
    assert "--kernel-trace --stats" in md and "--workload varlen_decode" in md
    d = tmp_path / "pmc"
    os.makedirs(d)
    k = "void pmqa::(anonymous namespace)::" + bench.COUNTED_KERNEL["spec_verify/fine"] + "(pmqa::LogitsArgs, int)"
    with open(d / "run_counter_collection.csv", "w", newline="") as f:
        w = csv.DictWriter(f, fieldnames=["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value",
                                          "Start_Timestamp", "End_Timestamp"])
        w.writeheader()
        for disp, busy in ((1, 3200.0), (2, 3200.0), (3, 6400.0)):
            for name, v in (("SQ_INSTS_MFMA", 100.0), ("SQ_VALU_MFMA_BUSY_CYCLES", busy)):
                # two rows per counter and dispatch (e.g. per XCD) are summed
                for _ in range(2):
                    w.writerow({"Dispatch_Id": disp, "Kernel_Name": k, "Counter_Name": name,
                                "Counter_Value": v / 2, "Start_Timestamp": 1000, "End_Timestamp": 21000})
    c = bench.counters_of(str(d), bench.COUNTED_KERNEL["spec_verify/fine"])
    assert c["SQ_INSTS_MFMA"] == 100.0 and c["SQ_VALU_MFMA_BUSY_CYCLES"] == 3200.0
    assert c["dispatches"] == 3 and c["duration_us"] == 20.0
    md = open(bench.write_counters_md(str(d), "spec_verify/fine", out_dir=str(tmp_path))).read()
    assert "Busy cycles per MFMA: 32.0" in md
