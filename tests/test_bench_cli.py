"""bench.py's command-line contract that needs no GPU: a run on several GPUs
is refused with a message (one GPU is measured; the path would shard without
an exchange inside attention), and the traffic record is keyed on the
kernel sources it was measured on."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_several_gpus_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                       text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    msg = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in msg["error"]


def test_traffic_reported_only_for_the_measured_sources(tmp_path, monkeypatch):
    """bench.py reports the committed HBM traffic record only while the
    kernel sources hash to the value the record was measured on, and null
    otherwise; the record's own arithmetic (counter KiB x calibration factor)
    is consistent."""
    sys.path.insert(0, ROOT)
    import bench

    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    assert rec["bytes_per_launch"] == rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    kib = rec["fetch_size_kib_per_dispatch"] * 1024 * rec["fetch_factor"]
    assert abs(kib - rec["read_bytes_per_launch"]) <= 1
    current = bench.kernel_source_hash()
    expect = rec["bytes_per_launch"] if rec["kernel_source_sha256"] == current else None
    assert bench.measured_traffic() == expect
    # a record of the current sources is used, one of other sources is not
    for sha, want in ((current, rec["bytes_per_launch"]), ("0" * 64, None)):
        f = tmp_path / f"traffic_{want}.json"
        f.write_text(json.dumps(dict(rec, kernel_source_sha256=sha)))
        monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
        assert bench.measured_traffic() == want
