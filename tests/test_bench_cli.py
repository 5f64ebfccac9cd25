"""bench.py's command line on a host without a GPU: the one-GPU rule and the workload list."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], capture_output=True,
                          text=True, timeout=120, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""                       # no JSON line for a run that did not happen


def test_unknown_workload_is_an_error():
    r = _run("--only", "stack,not_a_workload")
    assert r.returncode != 0
    assert "not_a_workload" in r.stderr


def test_help_lists_every_workload():
    r = _run("--help")
    assert r.returncode == 0
    for w in ("stack", "full_s8192", "sliding_s1024", "decode_b64", "decode_q8", "proj", "gemm_ref"):
        assert w in r.stdout
