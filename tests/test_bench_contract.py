"""bench.py's command-line contract, on the CPU: one GPU only (a request for
more exits with status 2 and says why, before anything touches a device), and
the defaults a plain run uses (N = 1, 200 timed steps after 20
warm-up steps, the gate/up pair layout)."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "single-GPU" in r.stderr
    assert r.stdout == ""


def test_defaults(monkeypatch):
    sys.path.insert(0, ROOT)
    import bench
    monkeypatch.setattr(sys, "argv", ["bench.py"])
    a = bench.parse()
    assert (a.gpus, a.steps, a.warmup, a.sets, a.layout) == (1, 200, 20, 4, 2)
    assert a.cpu_blocks > 0 and a.stack_layers == 40
