"""bench.py on the host: the single-GPU guard and the HBM traffic record."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert "one GPU" in line["error"]


def test_headline_traffic_record_matches_the_kernel_sources():
    """The measured HBM bytes of the headline kernel are reported only while its sources
    hash to the fingerprint taken with the counters; a kernel change must come with new
    counter passes (FETCH_SIZE, WRITE_SIZE) and a new record."""
    sys.path.insert(0, ROOT)
    import bench
    t = bench.measured_traffic("vit_s16_224", "fused")
    assert t is not None, "kernel sources changed since the HBM counters were taken"
    assert 0.9 * 28924416 < t < 1.5 * 28924416


def test_split_traffic_records_match_the_kernel_sources():
    sys.path.insert(0, ROOT)
    import bench
    for wl, algo in (("dense_64x64", 100794368), ("long_16k_bf16", 201850880)):
        t = bench.measured_traffic(wl, "split")
        assert t is not None, f"{wl}: split kernel sources changed since the counters were taken"
        assert algo < t < 2.5 * algo
