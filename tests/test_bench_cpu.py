"""bench.py on the CPU: the one-GPU guard, and how it takes the committed
HBM-traffic summaries (only for the kernel sources and launch plan they
were taken on)."""

import os
import subprocess
import sys

import bench

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(args, env_extra=None):
    env = dict(os.environ)
    env.update(env_extra or {})
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=120, env=env)


def test_more_than_one_gpu_exits_with_a_message():
    r = _run(["--gpus", "2"])
    assert r.returncode == 2
    assert "one GPU" in r.stdout + r.stderr
    r = _run([], {"WORLD_SIZE": "2"})
    assert r.returncode == 2


def test_traffic_summary_needs_matching_sources_and_plan():
    # the committed decode summary matches the committed sources and plan
    t = bench.load_traffic("llama2_7b_decode_fp16", "schedule=balanced partition=0 path=0")
    if t is not None:
        assert t["hbm_bytes_per_launch"] > 0
    # another launch plan, or a workload with no summary: no traffic figure
    assert bench.load_traffic("llama2_7b_decode_fp16", "schedule=fixed partition=512 path=1") is None
    assert bench.load_traffic("no_such_workload", "schedule=balanced partition=0 path=0") is None


def test_source_hash_covers_every_listed_file():
    h1 = bench.kernel_source_hash(bench.DECODE_SOURCES)
    h2 = bench.kernel_source_hash(bench.DECODE_SOURCES[:-1])
    assert h1 != h2 and len(h1) == 16
