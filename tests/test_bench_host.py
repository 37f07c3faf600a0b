"""Host-side checks of the benchmark's command line (no GPU needed)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "4"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_overrides_reach_the_workload():
    sys.path.insert(0, ROOT)
    import bench
    from sparse_attention_video_means_amd import synth
    old = sys.argv
    try:
        sys.argv = ["bench.py", "--workload", "stress", "--ck", "250", "--rho", "0.05"]
        args = bench.parse()
    finally:
        sys.argv = old
    wl = synth.WORKLOADS[args.workload].with_(ck=args.ck, rho=args.rho)
    assert (wl.ck, wl.rho, wl.budget) == (250, 0.05, int(0.05 * wl.n))
    assert bench.budget_for(wl, "cluster") == wl.budget
    assert bench.budget_for(wl, "global") == int(0.05 * wl.n * wl.n)
