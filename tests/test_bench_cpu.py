"""CPU checks of bench.py's accounting: the algorithmic FLOP and bytes behind
every roofline figure, and the turning of rocprofv3 counter readings into
bytes per launch.  Expected values are worked out by hand from the
definitions (2 (d_qk + d_v) FLOP per visible (query row, key) pair; each
visible cache row read once, plus q, O, LSE and the block-table or index
reads)."""
import csv
import json

import numpy as np
import pytest
import torch

import bench


def _dense_case(seqlens, s_q, h_q, causal=False, kv_fp8=False):
    return dict(s_q=s_q, d_qk=576, d_v=512, h_q=h_q, sparse=False, causal=causal, kv_fp8=kv_fp8,
                q=torch.zeros((len(seqlens), s_q, 1, 1)),
                cache_seqlens=torch.tensor(seqlens, dtype=torch.int32))


def test_tiny_workload_work():
    w = bench.algorithmic_work(_dense_case([64, 200], 1, 16))
    assert w["keys"] == 264
    assert w["flop"] == 16 * 264 * 2 * 1088 == 9_191_424
    kv = 264 * 1152
    q = 2 * 16 * 576 * 2
    o = 2 * 16 * (512 * 2 + 4)
    meta = (1 + 4) * 4 + 2 * 4  # block-table entries read, then the lengths
    assert w["kv_bytes"] == kv
    assert w["bytes"] == kv + q + o + meta == 373_916


def test_causal_mtp_work_counts_the_visible_keys_only():
    # 128 requests of 4096 tokens, two causal query tokens each: the first
    # sees 4095 keys, the second 4096
    w = bench.algorithmic_work(_dense_case([4096] * 128, 2, 128, causal=True))
    assert w["keys"] == 128 * (4095 + 4096)
    assert w["flop"] == 292_022_124_544
    # every cache row is read once per request, whatever the mask
    assert w["kv_bytes"] == 128 * 4096 * 1152
    # a request shorter than s_q: the earlier query tokens see nothing
    w = bench.algorithmic_work(_dense_case([1], 3, 1, causal=True))
    assert w["keys"] == 0 + 0 + 1


def test_fp8_rows_are_656_bytes():
    w = bench.algorithmic_work(_dense_case([100], 1, 64, kv_fp8=True))
    assert w["kv_bytes"] == 100 * 656
    assert w["flop"] == 100 * 64 * 2 * 1088


def test_sparse_work_counts_valid_indices_only():
    idx = torch.tensor([[[0, 5, -1, 64 * 4, 63]], [[-1, -1, 7, 200, 255]]], dtype=torch.int32)
    case = dict(s_q=1, d_qk=512, d_v=512, h_q=64, active_h_q=16, sparse=True, indices=idx,
                q=torch.zeros((2, 1, 64, 1)), kvcache=torch.zeros((4, 64, 1, 1)))
    w = bench.algorithmic_work(case)
    # rows 0..255 exist: 64*4 is out of range, -1 is invalid; 0, 5, 63 and
    # 7, 200, 255 remain
    assert w["keys"] == 3 + 3
    assert w["flop"] == 6 * 16 * 2 * 1024
    assert w["kv_bytes"] == 6 * 1024
    assert w["bytes"] == 6 * 1024 + 2 * 16 * 512 * 2 + 2 * 16 * (512 * 2 + 4) + idx.numel() * 4


def _write_counter_csv(path, counter, rows):
    with open(path, "w", newline="") as fh:
        wr = csv.writer(fh)
        wr.writerow(["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"])
        for i, (name, c, v) in enumerate(rows):
            wr.writerow([i, name, c, v])


def test_counter_ingestion_scales_by_the_copy_probe(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda k: str(tmp_path / f"traffic{k}.json"))
    probe_kib = bench.COPY_PROBE_BYTES / 1024
    split = "void mla::mla_splitkv<576, false, false, false, false>(mla::SplitKVParams)"
    neg = "void at::native::vectorized_elementwise_kernel<4, neg_kernel_cuda>(...)"
    fetch = tmp_path / "fetch.csv"
    write = tmp_path / "write.csv"
    # FETCH_SIZE reads half the bytes of the probe; the other counter of the
    # same pass and other kernels are ignored
    _write_counter_csv(fetch, "FETCH_SIZE", [
        (neg, "FETCH_SIZE", probe_kib / 2), (neg, "FETCH_SIZE", probe_kib / 2 + 3),
        (neg, "FETCH_SIZE", probe_kib / 2 - 1),
        (split, "FETCH_SIZE", 1000.0), (split, "FETCH_SIZE", 1200.0),
        (split, "TCC_HIT", 5.0), ("void mla::mla_combine<false>(mla::CombineParams)", "FETCH_SIZE", 77.0)])
    _write_counter_csv(write, "WRITE_SIZE", [
        (neg, "WRITE_SIZE", probe_kib), (split, "WRITE_SIZE", 300.0)])
    out = bench.ingest_counters(2, str(fetch), str(write), "cmd")
    assert out["fetch"]["dispatches"] == 2
    assert out["fetch"]["kib_per_launch"] == 1100.0
    assert out["fetch"]["probe_kib"] == probe_kib / 2  # the median of the probe readings
    assert out["fetch"]["probe_factor"] == 2.0
    assert out["fetch"]["bytes_per_launch"] == 1100 * 1024 * 2
    assert out["write"]["probe_factor"] == 1.0
    assert out["write"]["bytes_per_launch"] == 300 * 1024
    assert out["traffic_bytes_per_launch"] == 1100 * 1024 * 2 + 300 * 1024
    stored = json.load(open(tmp_path / "traffic2.json"))
    assert stored["kernel_hash"] == bench.kernel_hash() and stored["command"] == "cmd"


def test_counter_ingestion_needs_both_kernels(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda k: str(tmp_path / f"traffic{k}.json"))
    f = tmp_path / "f.csv"
    _write_counter_csv(f, "FETCH_SIZE", [("mla_splitkv<576>", "FETCH_SIZE", 1.0)])
    with pytest.raises(SystemExit):
        bench.ingest_counters(2, str(f), str(f), "cmd")


def test_counter_ingestion_takes_the_narrow_kernel(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "traffic_path", lambda k: str(tmp_path / f"traffic{k}.json"))
    probe_kib = bench.COPY_PROBE_BYTES / 1024
    narrow = "void mla::mla_narrow<512, true, false, 2>(mla::SplitKVParams)"
    neg = "void at::native::vectorized_elementwise_kernel<4, neg_kernel_cuda>(...)"
    f = tmp_path / "f.csv"
    w = tmp_path / "w.csv"
    _write_counter_csv(f, "FETCH_SIZE", [(neg, "FETCH_SIZE", probe_kib), (narrow, "FETCH_SIZE", 64.0)])
    _write_counter_csv(w, "WRITE_SIZE", [(neg, "WRITE_SIZE", probe_kib), (narrow, "WRITE_SIZE", 8.0)])
    out = bench.ingest_counters(5, str(f), str(w), "cmd")
    assert out["traffic_bytes_per_launch"] == (64 + 8) * 1024


def test_more_than_one_gpu_is_refused():
    """--gpus N with N > 1 exits with status 2 and says why, before any GPU work."""
    import subprocess
    import sys

    r = subprocess.run([sys.executable, bench.__file__, "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert msg["n_gpus"] == 2 and "one GPU only" in msg["error"]
