"""bench.py's command-line contract, on the CPU (no kernel runs here)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench(*args, env=None):
    return subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), *args], cwd=ROOT,
                          stdout=subprocess.PIPE, stderr=subprocess.PIPE, text=True, timeout=120, env=env)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = _bench("--gpus", "2")
    assert r.returncode == 2
    assert "one GPU" in r.stderr


def test_world_size_above_one_is_refused():
    env = dict(os.environ, WORLD_SIZE="4")
    r = _bench(env=env)
    assert r.returncode == 2


def test_help_lists_the_options():
    r = _bench("--help")
    assert r.returncode == 0
    for opt in ("--steps", "--warmup", "--workload", "--C", "--cold", "--tokens", "--split-ablation",
                "--staggered", "--calibrate-copy"):
        assert opt in r.stdout


def test_cpu_baseline_of_the_small_workload_has_a_one_thread_figure():
    """The oracle timing on the host: the small GDN workload (two heads) is
    timed with the thread pool and with one thread; every field present."""
    sys.path.insert(0, ROOT)
    import bench
    import workloads

    w = workloads.WORKLOADS["gdn_b1_h2_d32"]
    x = workloads.generate_workload(w)
    res = bench.cpu_baseline(x, w, w.B, 16)
    assert res["kind"] == "oracle" and res["unit"] == "us/token" and res["value"] > 0
    assert res["cores"] >= 1 and "first 16 tokens" in res["sample"]
    if res["cores"] > 2:
        one = res["one_thread"]
        assert one["cores"] == 1 and one["value"] > 0 and one["repeats"] >= 1
