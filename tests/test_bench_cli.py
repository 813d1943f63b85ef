"""bench.py's contract on the CPU: more than one GPU is refused with a
message, a host without a GPU is refused, and the roofline's measured traffic
is reported only while the committed counter summary matches the kernel
source it was taken on."""
from __future__ import annotations

import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def _run(*args):
    env = dict(os.environ, HIP_VISIBLE_DEVICES="")
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          timeout=300, env=env, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode != 0
    assert "ONE GPU" in r.stderr and "--gpus 2" in r.stderr


def test_no_gpu_is_refused_not_faked():
    import torch
    if torch.cuda.is_available():
        return
    r = _run("--steps", "1", "--warmup", "0")
    assert r.returncode != 0 and "no GPU" in r.stderr
    assert '"metric"' not in r.stdout


def test_traffic_follows_the_kernel_source(tmp_path, monkeypatch):
    import bench
    good = {"kernel_source_sha256_16": bench.kernel_source_hash(), "bytes_per_launch": 4294967296}
    f = tmp_path / "t.json"
    f.write_text(json.dumps(good))
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.measured_traffic() is not None
    f.write_text(json.dumps(dict(good, kernel_source_sha256_16="0" * 16)))
    assert bench.measured_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "missing.json"))
    assert bench.measured_traffic() is None
