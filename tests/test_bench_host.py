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


def test_committed_traffic_record_covers_launch_and_plan_code():
    """The record hashes the kernel source and the code that picks the variant and grid."""
    rec = json.load(open(os.path.join(ROOT, "profiles", "paged_decode_traffic.json")))
    srcs = set(rec["kernel_sources"])
    for f in ("decode.hip", "common.h", "kernels.h", "pagedattn.hip"):
        assert "paged_kv_cache_86_amd/csrc/" + f in srcs


def test_traffic_record_follows_the_sources(tmp_path):
    src = tmp_path / "kernel.src"
    src.write_bytes(b"kernel text")
    import hashlib
    good = {"kernel_sources": [os.path.relpath(str(src), ROOT)],
            "sha256": hashlib.sha256(b"kernel text").hexdigest(),
            "main_kernel": "k", "fetch_scale": 2.0, "write_scale": 1.0,
            "fetch_kib": {"k": 10.0, "merge": 99.0}, "write_kib": {"k": 1.0, "merge": 99.0}}
    rec = tmp_path / "traffic.json"
    rec.write_text(json.dumps(good))
    assert bench.counter_traffic(str(rec)) == 10 * 1024 * 2 + 1024
    src.write_bytes(b"kernel text, edited")
    assert bench.counter_traffic(str(rec)) is None
    assert bench.counter_traffic(str(tmp_path / "missing.json")) is None


def test_committed_traffic_record_matches_the_current_sources():
    """The committed counter record was taken from the decode sources as they stand, so the
    bench line carries roofline.traffic (an edit of those sources needs new counter runs)."""
    traffic = bench.counter_traffic(os.path.join(ROOT, "profiles", "paged_decode_traffic.json"))
    assert traffic is not None and traffic > 0
