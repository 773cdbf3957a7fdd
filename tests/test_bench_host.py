"""bench.py's host-side contract (no GPU needed).

* More than one GPU is refused with a message, before anything touches a GPU.
* The kernel source hash that ties the committed counter traffic to the
  kernel ignores comments and whitespace, and changes with the code.
"""
import importlib.util
import os
import subprocess
import sys

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


def _bench_module():
    spec = importlib.util.spec_from_file_location("bench_under_test", os.path.join(ROOT, "bench.py"))
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    return mod


def test_more_than_one_gpu_is_refused():
    res = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"], capture_output=True,
                         text=True, timeout=120)
    assert res.returncode == 2
    assert "one GPU only" in res.stderr
    assert res.stdout == ""


def test_kernel_hash_ignores_comments_and_whitespace():
    b = _bench_module()
    code = "int f(int x) {\n    return x + 1;   // one more\n}\n"
    assert b._code_only(code) == b._code_only("/* header */ int f(int x)\n{ return x + 1; }")
    assert b._code_only(code) != b._code_only(code.replace("x + 1", "x + 2"))
    assert len(b.kernel_source_hash()) == 16
