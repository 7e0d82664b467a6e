"""The benchmark's command-line contract, checked without a GPU: more than
one GPU is refused with a message (this build measures one GPU), and the
counter summary refuses folders without counter rows."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, cwd=ROOT, timeout=300)


def test_more_than_one_gpu_is_refused():
    r = _bench("--gpus", "2", "--steps", "1", "--warmup", "0")
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout.strip() == ""


def test_counter_summary_needs_counter_rows(tmp_path):
    r = _bench("--summarize-counters", str(tmp_path), str(tmp_path))
    assert r.returncode != 0
    assert "no FETCH_SIZE rows" in (r.stdout + r.stderr)
