"""Host-side parts of the measurement, on the CPU: the bench's algorithmic byte
count (the numerator of every GB/s and roofline figure it prints) against the
oracle's element-by-element count, the rocprofv3 counter summary's scaling by
a copy of known size, the traffic file's source check, and the one-GPU guard."""
import csv
import os
import subprocess
import sys

import numpy as np
import pytest

import bench
import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.parametrize("hq,hkv,d,ctx,cap,sparsity", [
    (8, 2, 128, [200, 77, 0], 224, 40),       # ragged rows, one empty, one inside its third group
    (4, 1, 64, [31, 32, 33], 64, 60),        # around one key group
    (8, 8, 64, [150], 160, 0),              # one query head per KV head, no pruning
])
def test_bench_decode_bytes_equal_oracle_count(orc, hq, hkv, d, ctx, cap, sparsity):
    wl = W.custom(f"bytes{hq}{d}", 31 + hq + d, len(ctx), hq, hkv, d, ctx, cap, "bf16",
                  log_uniform_key_scales=True)
    a, b = W.transforms(wl)
    c = orc.Cache(wl.batch, wl.hkv, wl.d, wl.cap)
    k, v = W.prefill_kv(wl)
    c.append(k, v, b, list(wl.ctx))
    keep = orc.keep_count(d, sparsity)
    _, idx = orc.queries(W.queries(wl), a, wl.hkv, keep)
    want = int(c.decode_bytes(idx).astype(np.int64).sum())
    assert bench.decode_bytes(idx, c.lengths, wl.hkv, wl.d, keep) == want


def _write_csv(path, header, rows):
    with open(path, "w", newline="") as f:
        w = csv.writer(f)
        w.writerow(header)
        w.writerows(rows)


def test_counter_summary_scales_by_the_copy(tmp_path, capsys):
    """FETCH_SIZE of a 64 MiB device copy reading 32768 KiB gives the factor 2.0,
    and the target kernel's average per dispatch is scaled by it."""
    run = tmp_path / "host" / "1"
    run.mkdir(parents=True)
    hdr = ["Dispatch_Id", "Kernel_Name", "Counter_Name", "Counter_Value"]
    rows = [[1, "decode4_kernel<128, false>", "FETCH_SIZE", 1000.0],
            [2, "decode4_kernel<128, false>", "FETCH_SIZE", 3000.0],
            [3, "__amd_rocclr_copyBuffer", "FETCH_SIZE", 32768.0],
            [4, "combine_kernel<128>", "FETCH_SIZE", 7.0]]
    _write_csv(run / "run_counter_collection.csv", hdr, rows)
    _write_csv(run / "run_kernel_stats.csv",
               ["Name", "Calls", "TotalDurationNs", "AverageNs", "Percentage", "MinNs", "MaxNs"],
               [["decode4_kernel<128, false>", 2, 60000, 30000, 90.0, 29000, 31000]])
    bench.summarize_rocprof(str(tmp_path), "decode4_kernel", 64)
    out = capsys.readouterr().out
    assert "2 dispatches of /decode4_kernel/" in out
    assert "FETCH_SIZE_avg_kib_per_dispatch: 2000.0" in out
    assert "factor 2.0000" in out
    assert "FETCH_SIZE_bytes_per_dispatch_scaled: 4096000" in out
    assert "30.00" in out   # the kernel statistics in microseconds


def test_recorded_traffic_needs_the_same_kernel_sources(monkeypatch):
    """The committed counter summary is used only while its source hash is that of the
    decode kernels as they stand; any other code gives None."""
    fields = {}
    for line in open(bench.TRAFFIC_FILE):
        if ":" in line and not line.startswith((" ", "#")):
            k, v = line.split(":", 1)
            fields[k.strip()] = v.strip()
    assert int(fields["traffic_bytes_per_launch"]) > int(fields["algorithmic_bytes_per_launch"])
    if fields["source_hash"] == bench.kernel_source_hash():
        assert bench.recorded_traffic() == int(fields["traffic_bytes_per_launch"])
    monkeypatch.setattr(bench, "kernel_source_hash", lambda *a, **k: "0000000000000000")
    assert bench.recorded_traffic() is None


def test_kernel_source_hash_ignores_comments_and_layout():
    def read(rel):
        return open(os.path.join(ROOT, rel), encoding="utf-8").read()
    h = bench.kernel_source_hash(read=read)
    assert h == bench.kernel_source_hash()
    reflowed = bench.kernel_source_hash(
        read=lambda rel: "// a comment\n" + read(rel).replace("\n", "\n\n  ") + "\n/* more */")
    assert reflowed == h
    changed = bench.kernel_source_hash(
        read=lambda rel: read(rel).replace("kChunk4", "kChunkX", 1) if rel.endswith("dqk_decode4.hip") else read(rel))
    assert changed != h


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""
