"""The build entry point compiles the HIP library and imports the package (CPU only)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))


@pytest.mark.skipif(not os.path.exists("/opt/rocm/bin/hipcc"), reason="hipcc not installed")
def test_graft_build_entry_compiles_and_imports():
    code = "import __graft_entry__ as g; g.build()"
    r = subprocess.run([sys.executable, "-c", code], cwd=ROOT, capture_output=True, text=True,
                       timeout=900)
    assert r.returncode == 0, r.stderr[-2000:]
    assert "imports" in r.stdout


def test_bench_refuses_more_than_one_gpu():
    """The measurement runs on one GPU; asking for more exits with a message before
    any device work."""
    r = subprocess.run([sys.executable, "bench.py", "--gpus", "2"], cwd=ROOT, capture_output=True,
                       text=True, timeout=300)
    assert r.returncode == 2
    assert "one GPU only" in r.stderr
