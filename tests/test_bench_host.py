"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the kernel
source hash, and the rule that the counter-derived traffic figure is reported
only while it was taken on the current kernel sources."""
import json
import os
import shutil
import subprocess
import sys

import bench
from synthetic import workloads as W

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")], capture_output=True, text=True,
                       timeout=120, env=env)
    assert r.returncode == 2


def _copy_sources(tmp_path):
    d = tmp_path / "csrc"
    shutil.copytree(bench.KERNEL_SRC_DIR, d)
    return d


def test_source_hash_covers_every_source_and_header(tmp_path, monkeypatch):
    d = _copy_sources(tmp_path)
    monkeypatch.setattr(bench, "KERNEL_SRC_DIR", str(d))
    h0 = bench.kernel_source_hash()
    assert h0 == bench.kernel_source_hash()
    names = sorted(n for n in os.listdir(d) if n.endswith((".hip", ".h")))
    assert len(names) >= 4
    for name in names:
        p = d / name
        text = p.read_bytes()
        p.write_bytes(text + b"\n")
        assert bench.kernel_source_hash() != h0, f"{name} is not covered by the hash"
        p.write_bytes(text)
    assert bench.kernel_source_hash() == h0
    # Files that are not sources do not count.
    (d / "notes.txt").write_text("x")
    assert bench.kernel_source_hash() == h0
    # A renamed file changes the hash even with the same bytes.
    os.rename(d / names[0], d / ("z" + names[0]))
    assert bench.kernel_source_hash() != h0


def _traffic_file(tmp_path, **fields):
    t = {"workload": W.HEADLINE.name, "kernel_source_sha256": bench.kernel_source_hash(),
         "hbm_bytes_per_launch": 123456789}
    t.update(fields)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(t))
    return p


def test_traffic_reported_when_taken_on_these_sources(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(_traffic_file(tmp_path)))
    assert bench.load_traffic(W.HEADLINE.name) == 123456789


def test_traffic_null_on_other_sources_workload_or_bad_file(tmp_path, monkeypatch):
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(_traffic_file(tmp_path, kernel_source_sha256="0" * 64)))
    assert bench.load_traffic(W.HEADLINE.name) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(_traffic_file(tmp_path)))
    assert bench.load_traffic("nn_1024") is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.load_traffic(W.HEADLINE.name) is None
    bad = tmp_path / "bad.json"
    bad.write_text("{not json")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(bad))
    assert bench.load_traffic(W.HEADLINE.name) is None


def test_committed_traffic_summary_is_for_the_headline_workload():
    with open(bench.TRAFFIC_FILE) as f:
        t = json.load(f)
    assert t["workload"] == W.HEADLINE.name
    assert t["algorithmic_bytes_per_launch"] == W.HEADLINE.algorithmic_bytes
    # Read and write bytes, each a copy-calibrated counter reading, add up.
    assert t["hbm_bytes_per_launch"] == t["hbm_read_bytes_per_launch"] + t["hbm_write_bytes_per_launch"]


def test_spread_of_per_call_times():
    per = [5.0, 1.0, 4.0, 2.0, 3.0, 9.0, 7.0, 8.0, 6.0, 10.0]
    s = bench.spread(per)
    assert s == {"median": 6.0, "min": 1.0, "p90": 10.0, "max": 10.0, "first": 5.0, "last": 10.0}
    assert bench.spread([2.5]) == {"median": 2.5, "min": 2.5, "p90": 2.5, "max": 2.5, "first": 2.5, "last": 2.5}
