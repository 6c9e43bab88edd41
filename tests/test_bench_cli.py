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


def test_traffic_record_matches_current_sources():
    sys.path.insert(0, ROOT)
    import bench

    with open(bench.TRAFFIC_FILE) as fh:
        rec = json.load(fh)
    # the committed counter record belongs to the attention kernel as it is now
    assert rec["kernel_source_sha256"] == bench.kernel_source_hash()
    assert bench.measured_traffic() == rec["bytes_per_launch"]
    assert rec["bytes_per_launch"] == rec["read_bytes_per_launch"] + rec["write_bytes_per_launch"]
    kib = rec["fetch_size_kib_per_dispatch"] * 1024 * rec["fetch_factor"]
    assert abs(kib - rec["read_bytes_per_launch"]) <= 1
