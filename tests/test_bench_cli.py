"""bench.py's command-line contract that needs no GPU: more than one GPU is
refused with a message and exit status 2, before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], cwd=ROOT,
                       capture_output=True, text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and "--gpus 2" in r.stderr
    assert r.stdout.strip() == ""  # no JSON line


def test_csv_results_file(tmp_path):
    """The results file of the pages' benchmark assignment: a header, one row
    per length, "OOM" kept as text."""
    import csv

    import bench
    path = tmp_path / "sweep.csv"
    bench.write_csv(str(path), ["L", "time_ms", "mem_GB"], [[4096, 0.03, 0.008], [131072, "OOM", "OOM"]])
    rows = list(csv.reader(open(path)))
    assert rows == [["L", "time_ms", "mem_GB"], ["4096", "0.03", "0.008"], ["131072", "OOM", "OOM"]]
