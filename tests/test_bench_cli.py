"""bench.py's command line on a machine without a GPU: asking for more than
one GPU is refused with a JSON message and exit status 2 before anything
touches a device, and --help lists every row's mode."""
import json
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _run(*args):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args],
                          capture_output=True, text=True, timeout=300, cwd=ROOT)


def test_more_than_one_gpu_is_refused():
    r = _run("--gpus", "2")
    assert r.returncode == 2
    line = json.loads(r.stdout.strip().splitlines()[-1])
    assert line["n_gpus"] == 2 and "one GPU" in line["error"]


def test_help_names_every_mode():
    r = _run("--help")
    assert r.returncode == 0
    for flag in ("--prefill", "--window", "--fp8", "--cow", "--step", "--copy-calibration"):
        assert flag in r.stdout


def test_cpu_baseline_runs_on_the_small_workload():
    """The oracle's timed leg (all cores, then one core), on the host alone,
    plain, with a window and with FP8 pools."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads
    w = workloads.make(1, seed=1, poison=False)
    for window, fp8 in ((0, None), (8, None), (0, (4.0 / 448, 4.0 / 448))):
        kv = bench.kv_bytes_per_step(w, window) // (w.elem_bytes if fp8 else 1)
        all_tbps, cores, one_tbps, sample = bench.cpu_baseline(w, 0.4, kv, window, fp8)
        assert all_tbps > 0 and one_tbps > 0 and 1 <= cores <= 16
        assert "one core" in sample
