"""bench.py's host-side contract, without a GPU: the one-GPU refusal and the rule that the
reported HBM traffic is null once the kernel source differs from the one the counters were
taken on."""
import json
import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True, text=True,
                          env=env, cwd=ROOT, timeout=120)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_a_distributed_launch_is_refused_too():
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2
    assert "error" in json.loads(r.stdout.strip().splitlines()[-1])


def test_traffic_is_read_only_for_the_profiled_source(tmp_path, monkeypatch):
    sha = bench.source_sha(bench.ATTN_SRC)
    f = tmp_path / "traffic.txt"
    f.write_text(f"# summary\nkernel_source_sha256_16: {sha}\nhbm_bytes_per_launch: 1.5e+09\n")
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(f))
    assert bench.read_traffic() == 1.5e9
    f.write_text("kernel_source_sha256_16: 0000000000000000\nhbm_bytes_per_launch: 1.5e+09\n")
    assert bench.read_traffic() is None
    monkeypatch.setattr(bench, "TRAFFIC_FILE", str(tmp_path / "absent.txt"))
    assert bench.read_traffic() is None

