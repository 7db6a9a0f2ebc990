"""Host logic of bench.py, on the CPU: the one-GPU guard, the staleness rule
of the counter-measured HBM traffic, and the committed traffic records."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr


def test_traffic_record_goes_null_when_a_source_changes(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "ROOT", str(tmp_path))
    src = tmp_path / "k.hip"
    src.write_text("__global__ void k() {}\n")
    (tmp_path / "profiles").mkdir()
    rec = {"w:gemm": {"bytes_per_launch": 1234, "sources": ["k.hip"],
                      "sources_sha256": bench.sources_sha256(["k.hip"])}}
    (tmp_path / "profiles" / "hbm_traffic.json").write_text(json.dumps(rec))
    assert bench.traffic_record("w:gemm") == 1234
    assert bench.traffic_record("w:act") is None          # no record for that kernel
    src.write_text("__global__ void k() { /* changed */ }\n")
    assert bench.traffic_record("w:gemm") is None          # counters older than the source


def test_committed_traffic_records_are_well_formed():
    recs = json.load(open(os.path.join(ROOT, "profiles", "hbm_traffic.json")))
    assert recs
    for key, rec in recs.items():
        workload, kernel = key.split(":")
        assert workload and kernel
        assert rec["bytes_per_launch"] > 0
        assert abs(rec["bytes_per_launch"] - rec["read_bytes"] - rec["write_bytes"]) <= 1   # each part rounded
        assert os.path.exists(os.path.join(ROOT, "profiles", rec["summary"])), key
        for s in rec["sources"]:
            assert os.path.exists(os.path.join(ROOT, s)), (key, s)


def test_stream_windows_stay_inside_the_buffers():
    """The live ceilings' plain stream takes launch w's bytes at offset
    w * size of each buffer: every window of every workload's transform
    stays inside both buffers, and streams outside the measured range (under
    8 MiB, over 1 GiB, sizes the probe refuses) get no windows."""
    act_reads = [4096 * 14336 * 2, 2048 * 4096 * 2, 8192 * 3072 * 2, 8 << 20, 1 << 30, 3 * (8 << 20) + 64]
    for rb in act_reads:
        wb = rb // 4
        n = bench.stream_windows(rb, wb)
        assert 1 <= n <= 64, rb
        assert n * rb <= bench.STREAM_SRC_BYTES and n * wb <= bench.STREAM_DST_BYTES, rb
    for rb, wb in [(8192 * 2 * 8, 8192 * 4), ((1 << 30) + 64, 1 << 28), (0, 0), (16 << 20, 0),
                   ((16 << 20) + 8, (4 << 20) + 2), (16 << 20, 3 << 20)]:
        assert bench.stream_windows(rb, wb) == 0, (rb, wb)
