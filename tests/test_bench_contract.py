"""CPU checks of bench.py's contract: one GPU only, and the byte formulas of
the metric (logical and algorithmic bytes per step)."""
import os
import subprocess
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
sys.path.insert(0, ROOT)

import bench  # noqa: E402
import workloads  # noqa: E402


@pytest.mark.parametrize("argv,env", [(["--gpus", "2"], {}), (["--gpus", "8"], {}),
                                      ([], {"WORLD_SIZE": "2"})])
def test_more_than_one_gpu_exits_with_a_message(argv, env):
    e = dict(os.environ, **env)
    r = subprocess.run([sys.executable, os.path.join(ROOT, "bench.py")] + argv, capture_output=True,
                       text=True, env=e, timeout=120)
    assert r.returncode == 2
    assert "one GPU" in r.stderr
    assert r.stdout == ""


def test_v3_byte_counts():
    wl = workloads.config("v3")
    N = wl.T * wl.K                      # the V3 routing masks nothing
    bc = bench.byte_counts(wl, N)
    H, nb = wl.H, wl.H // 128
    assert bc["dispatch_logical"] == N * (H + 4 * nb) == 484_442_112
    assert bc["combine_logical"] == N * H * 2 == 939_524_096
    # the rows moved dominate the algorithmic bytes; metadata adds < 1%
    assert 0 < bc["dispatch_alg"] - (wl.T * H * 2 + bc["dispatch_logical"]) < 0.01 * bc["dispatch_alg"]
    assert bc["combine_alg"] == N * H * 2 + wl.T * H * 2 + wl.T * wl.K * 8


def test_bf16_byte_counts_have_no_scales():
    wl = workloads.config("skewed")
    bc = bench.byte_counts(wl, 1000)
    assert bc["dispatch_logical"] == 1000 * wl.H * 2
