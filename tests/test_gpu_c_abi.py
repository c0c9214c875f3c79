"""The C ABI from plain C: tests/c_abi_driver (built with the library) runs
layout -> dispatch (FP8 and BF16) -> counts -> combine, and the
allocation-free low-latency dispatch twice in a row, through the HIP runtime
only, and compares every output with the CPU oracle byte for byte."""
import os
import subprocess

import pytest

pytestmark = pytest.mark.gpu

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
DRIVER = os.path.join(ROOT, "tests", "c_abi_driver")


def test_c_driver_matches_the_oracle():
    torch = pytest.importorskip("torch")
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    assert os.path.exists(DRIVER), "tests/c_abi_driver is missing: run __graft_entry__.build()"
    r = subprocess.run([DRIVER], capture_output=True, text=True, timeout=120)
    print(r.stdout)
    assert r.returncode == 0, r.stdout + r.stderr
    assert "c abi driver: ok" in r.stdout
