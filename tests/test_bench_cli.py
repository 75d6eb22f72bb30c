"""bench.py's command-line contract on the CPU: a request for more than one GPU
is refused with a message (the library measures one GPU) before any device work."""
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode != 0
    assert "one GPU" in res.stderr and res.stdout == ""


def test_help_lists_the_options():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--help"],
                         capture_output=True, text=True, timeout=60)
    assert res.returncode == 0
    for opt in ("--gpus", "--steps", "--warmup", "--workload", "--n-feat", "--impl", "--peaks", "--no-fp32-compare"):
        assert opt in res.stdout


def test_source_check_ignores_comments_only():
    sys.path.insert(0, ROOT)
    import bench
    a = "int f(int x) {\n  return x + 1;  // add one\n}\n"
    b = "/* header\n   text */\nint f(int x) {\n\n  // a new comment\n  return x + 1;\n}\n"
    c = "int f(int x) {\n  return x + 2;\n}\n"
    assert bench.code_text(a) == bench.code_text(b)
    assert bench.code_text(a) != bench.code_text(c)
