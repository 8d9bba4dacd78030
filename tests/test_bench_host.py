"""bench.py on the host: it refuses more than one GPU before touching one, and reports the
counter-derived HBM traffic only while the kernel sources still hash to the recorded value."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    p = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       stdout=subprocess.PIPE, stderr=subprocess.STDOUT, text=True, timeout=120)
    assert p.returncode != 0
    assert "one GPU" in p.stdout


def test_traffic_record_follows_the_sources(tmp_path):
    src = tmp_path / "kernel.src"
    src.write_bytes(b"kernel text")
    import hashlib
    good = {"kernel_sources": [os.path.relpath(str(src), ROOT)],
            "sha256": hashlib.sha256(b"kernel text").hexdigest(),
            "decode_bytes_per_launch": 12345}
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps(good))
    assert bench.counter_traffic(str(rec)) == 12345
    src.write_bytes(b"kernel text, edited")
    assert bench.counter_traffic(str(rec)) is None
    assert bench.counter_traffic(str(tmp_path / "missing.json")) is None
