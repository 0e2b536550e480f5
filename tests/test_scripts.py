"""The repository's entry scripts without a GPU: they compile, and bench.py
refuses more than one GPU with a message."""
import os
import py_compile
import subprocess
import sys

from conftest import ROOT


def test_scripts_compile():
    for name in ("bench.py", "__graft_entry__.py"):
        py_compile.compile(os.path.join(ROOT, name), doraise=True)


def test_bench_refuses_several_gpus():
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py"), "--gpus", "2"],
                       capture_output=True, text=True, timeout=120, cwd=ROOT)
    assert r.returncode != 0
    assert "one GPU" in (r.stdout + r.stderr)
