"""CPU checks of bench.py's contract points that need no GPU: more than one
GPU is refused with a message, and the committed HBM-traffic record is used
only while it was taken on the current kernel source."""
import json
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_traffic_record_follows_the_source_hash(monkeypatch):
    import bench
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        rec = json.load(f)
    for name, srcs in (("long", bench.KERNEL_SRC), ("prefill", bench.KERNEL_SRC),
                       ("attn", bench.ATTN_SRC), ("attn_long", bench.ATTN_SRC)):
        ent = rec[name]
        monkeypatch.setattr(bench, "kernel_source_hash", lambda s=None, h=ent["kernel_source_hash"]: h)
        assert bench.measured_traffic(name, srcs) == ent["bytes_per_launch"]
        monkeypatch.setattr(bench, "kernel_source_hash", lambda s=None: "0" * 16)
        assert bench.measured_traffic(name, srcs) is None


@pytest.mark.parametrize("name", ["long", "prefill", "attn", "attn_long"])
def test_traffic_record_is_consistent(name):
    with open(os.path.join(ROOT, "profiles", "traffic.json")) as f:
        ent = json.load(f)[name]
    kib = 1024
    if name in ("long", "prefill"):
        got = (ent["fetch_size_kib_per_dispatch"] * ent["fetch_scale"]
               + ent["write_size_kib_per_dispatch"] * ent["write_scale"]) * kib
    else:
        got = ((ent["split_fetch_size_kib_per_dispatch"] + ent["combine_fetch_size_kib_per_dispatch"])
               * ent["fetch_scale"]
               + (ent["split_write_size_kib_per_dispatch"] + ent["combine_write_size_kib_per_dispatch"])
               * ent["write_scale"]) * kib
    assert abs(got - ent["bytes_per_launch"]) <= 1e-4 * ent["bytes_per_launch"]
    # traffic can exceed the algorithmic bytes (partials, partial lines) but never undercut
    # them by more than rounding of the counters
    assert ent["bytes_per_launch"] >= 0.999 * ent["algorithmic_bytes_per_launch"]
