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


def test_committed_traffic_figures_match_the_kernel_sources():
    """profiles/traffic.json holds the counter-measured HBM bytes that the
    bench line reports as `traffic`; each entry names a hash of the sources
    its kernels were built from, and the bench drops a figure whose hash no
    longer matches.  Every committed entry is current, and every kernel set
    the bench looks up has an entry."""
    import importlib.util
    import json
    spec = importlib.util.spec_from_file_location("bench_mod", BENCH)
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    with open(bench.TRAFFIC_FILE) as f:
        traffic = json.load(f)
    assert set(traffic) == set(bench.KERNEL_SOURCES)
    for name, entry in traffic.items():
        assert entry["kernel_sha"] == bench.kernel_sha(name), f"{name}: re-take its counters"
        assert abs(entry["bytes_per_launch"] - entry["fetch_bytes"] - entry["write_bytes"]) <= 1
        assert bench.traffic_for(name) == float(entry["bytes_per_launch"])
