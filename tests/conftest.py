import os
import sys

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
if ROOT not in sys.path:
    sys.path.insert(0, ROOT)


def pytest_configure(config):
    config.addinivalue_line("markers", "gpu: needs an MI355X (gfx950) GPU")
    config.addinivalue_line("markers", "slow: CPU test that takes more than a few seconds")


def gpu_available() -> bool:
    try:
        import torch
        return torch.cuda.is_available()
    except Exception:
        return False


@pytest.fixture(scope="session")
def ep():
    """The HIP library's Python binding (fails loudly if the library is missing)."""
    import combine_get_dispatch_scan_amd as m
    m.load()
    return m


def grad_w_rel_bound(H: int) -> float:
    """Worst-case relative error of combine_backward's grad_w against the exact
    dot product, as a multiple of sum_j |g_j y_j|.

    The kernel reduces each dot product in a fixed order: a lane's fp32 fma
    chain over 8 channels in each of its ceil(ceil(H/512)/8) wave steps, a
    6-level xor-shuffle tree over the 64 lanes, then 7 sequential adds of the
    8 waves' partial sums.  The bf16 x bf16 products are exact in fp32, so a
    term passes through at most d = 8*ceil(ceil(H/512)/8) + 13 roundings, and
    the standard recursive-summation bound gives gamma_d = d*u/(1-d*u) with
    u = 2^-24."""
    steps = -(-H // 512)
    d = 8 * (-(-steps // 8)) + 13
    u = 2.0 ** -24
    return d * u / (1.0 - d * u)
