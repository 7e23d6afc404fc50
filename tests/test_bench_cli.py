"""bench.py's command line on the CPU: more than one GPU is refused with a
message before anything touches a device, and the help lists the contract's
flags."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "exactly one GPU" in r.stderr and r.stdout == ""


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="2")
    r = _run(env=env)
    assert r.returncode == 2 and "exactly one GPU" in r.stderr


def test_help_lists_the_contract_flags():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ["--gpus", "--steps", "--warmup", "--workload"]:
        assert flag in r.stdout


def test_traffic_is_dropped_once_the_lm_head_source_changes(tmp_path, monkeypatch):
    # roofline.traffic comes from stored counters only while the hash of the
    # LM-head source (the kernel file and the device helpers it inlines)
    # matches the one recorded with them
    import json
    sys.path.insert(0, ROOT)
    import bench
    srcs = [tmp_path / "k.hip", tmp_path / "h.hpp"]
    srcs[0].write_text("kernel v1\n")
    srcs[1].write_text("helpers v1\n")
    monkeypatch.setattr(bench, "LMHEAD_SRCS", [str(p) for p in srcs])
    rec = {"c2": {"workload": "c2", "kernel_source_sha": bench._sha([str(p) for p in srcs]),
                  "fetch_kib": 100.0, "fetch_factor": 2.0, "write_kib": 10.0, "write_factor": 1.0}}
    counters = tmp_path / "counters.txt"
    counters.write_text("# header\n" + json.dumps(rec) + "\n")
    monkeypatch.setattr(bench, "COUNTERS_FILE", str(counters))
    assert bench._traffic("c2") == (100.0 * 2.0 + 10.0) * 1024.0
    assert bench._traffic("c5") is None
    srcs[1].write_text("helpers v2\n")          # a helper changed: the counters are stale
    assert bench._traffic("c2") is None
