"""Host-side logic of bench.py, on the CPU: the one-GPU guard, the kernel
code hash, and the rule that the counter-derived traffic figure is reported
only while the built kernel's machine code is the code it was taken on."""
import hashlib
import json
import os
import subprocess
import sys

import pytest

import bench
import fp32_gemm_nn_amd as mg
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


HEADLINE_KERNEL = r"sgemm_mfma32INS_7TileCfgILi256ELi256ELi32ELi4ELi2ELi1ELi0ELb0ELb0ELb0ELb0EEELb0ELb0ELb0E"


def _built():
    if not os.path.exists(mg.library_path):
        pytest.skip("library not built")


def test_kernel_code_hash_is_the_kernels_machine_code():
    """The traffic record is tied to one kernel's gfx950 machine code, read from
    the built library's code objects."""
    _built()
    from fp32_gemm_nn_amd import codeobj

    code = codeobj.kernel_code(mg.library_path)
    assert len(code) > 200
    sym = codeobj.find_symbol(mg.library_path, HEADLINE_KERNEL)
    h = bench.kernel_code_hash(sym)
    assert h == hashlib.sha256(code[sym]).hexdigest()
    # Whole instructions, and a different kernel hashes differently.
    assert len(code[sym]) % 4 == 0 and len(code[sym]) > 4096
    other = next(n for n in code if n != sym and "sgemm_mfma32" in n)
    assert bench.kernel_code_hash(other) != h
    assert bench.kernel_code_hash("_Z_no_such_kernel") is None


def _traffic_file(tmp_path, **fields):
    from fp32_gemm_nn_amd import codeobj

    sym = codeobj.find_symbol(mg.library_path, HEADLINE_KERNEL)
    t = {"workload": W.HEADLINE.name, "kernel_symbol": sym, "kernel_code_sha256": bench.kernel_code_hash(sym),
         "hbm_bytes_per_launch": 123456789}
    t.update(fields)
    p = tmp_path / "traffic.json"
    p.write_text(json.dumps(t))
    return p


def test_traffic_reported_when_taken_on_this_kernel_code(tmp_path, monkeypatch):
    _built()
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(_traffic_file(tmp_path)))
    assert bench.load_traffic(W.HEADLINE.name) == 123456789


def test_traffic_null_on_other_code_workload_or_bad_file(tmp_path, monkeypatch):
    _built()
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(_traffic_file(tmp_path, kernel_code_sha256="0" * 64)))
    assert bench.load_traffic(W.HEADLINE.name) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(_traffic_file(tmp_path, kernel_symbol="_Z_no_such_kernel")))
    assert bench.load_traffic(W.HEADLINE.name) is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(_traffic_file(tmp_path, kernel_symbol=None)))
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
