"""bench.py's command-line contract on the CPU: more than one GPU is refused
with a message before any GPU work; the kernel-source digest that ties the
committed counter summaries to the kernels ignores comments and layout."""

import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)


def test_more_than_one_gpu_is_refused_with_a_message():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr and r.stdout == ""


def test_digest_ignores_comments_and_layout():
    import bench
    a = "int f(int x) {  // the answer\n  return x + 1; /* one\n more */\n}\n"
    b = "int f(int x) { return x + 1; }"
    c = "int f(int x) { return x + 2; }"
    assert bench._code_only(a) == bench._code_only(b) != bench._code_only(c)
    d = bench.kernel_source_digest()
    assert len(d) == 64 and d == bench.kernel_source_digest()
