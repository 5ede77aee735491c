"""bench.py's command line on the CPU: it measures one GPU and says so when
asked for more (no GPU is touched before that check)."""
import os
import subprocess
import sys

BENCH = os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py")


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, BENCH, "--gpus", "2"], capture_output=True, text=True,
                       timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_a_second_rank_is_refused():
    env = dict(os.environ, RANK="1", WORLD_SIZE="2")
    r = subprocess.run([sys.executable, BENCH], capture_output=True, text=True, timeout=120,
                       env=env)
    assert r.returncode == 2
    assert "single process" in r.stderr
