"""CPU checks of bench.py's contract: one GPU only, and the byte formulas of
the metric (logical and algorithmic bytes per step)."""
import os
import subprocess
import sys

import numpy as np
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


def test_bf16_ulp_distance():
    u = lambda *v: np.array(v, dtype=np.uint16)
    assert bench.bf16_ulp_distance(u(0x3F80), u(0x3F80)) == 0
    assert bench.bf16_ulp_distance(u(0x3F80), u(0x3F81)) == 1
    assert bench.bf16_ulp_distance(u(0x0000), u(0x8000)) == 0       # +0 and -0 meet
    assert bench.bf16_ulp_distance(u(0x0001), u(0x8001)) == 2       # across zero
    assert bench.bf16_ulp_distance(u(0xBF80), u(0xBF81)) == 1
    assert bench.bf16_ulp_distance(u(0x3F80, 0x4000), u(0x3F80, 0x4003)) == 3


def _gpu_like(ref, N):
    """The oracle's own results, shaped like the bench's snapshot of a step."""
    return {"ntpe": ref["num_tokens_per_expert"].copy(), "ntpp": ref["num_tokens_per_partition"].copy(),
            "itip": ref["is_token_in_partition"].copy(), "ninv": ref["num_invalid"],
            "slot": ref["slot"].copy(), "recv": ref["recv_x"][:N].copy(),
            "scales": ref["recv_scales"][:N].copy() if ref["recv_scales"] is not None else None,
            "out": ref["out"].copy()}


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_parity_verdict_on_the_oracle_itself_and_planted_mistakes(name):
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    y = workloads.expert_outputs(wl, N)
    _, n, ref = bench.cpu_baseline(wl, idx, w, x, y, 1)
    assert n == N
    v = bench.parity_verdict(_gpu_like(ref, N), ref, N, wl.use_fp8)
    assert all(v[k] == "bit-exact" for k in ("layout", "slot", "recv_rows", "combine"))
    assert v["combine_max_ulp"] == 0
    # planted differences are reported
    g = _gpu_like(ref, N)
    g["slot"][0, 0] += 1
    g["recv"][N - 1, -1] ^= 1
    g["out"][3, 5] += 1
    g["ntpe"][0] += 1
    v = bench.parity_verdict(g, ref, N, wl.use_fp8)
    assert v["slot"] == v["recv_rows"] == v["layout"] == "MISMATCH"
    assert v["combine_max_ulp"] == 1 and v["combine"] == "within 1 ulp"
    if wl.use_fp8:
        g["scales"][0, 0] = np.nextafter(g["scales"][0, 0], np.float32(np.inf))
        assert bench.parity_verdict(g, ref, N, True)["recv_scales"] == "MISMATCH"


@pytest.mark.parametrize("wl", [workloads.config("tiny"),
                                workloads.Workload("bench_mt_fp8", 300, 512, 32, 4, 8, True, 91, "softmax")],
                         ids=["tiny-bf16", "fp8"])
def test_threaded_oracle_leg_matches_the_single_thread_run(wl):
    """The threaded CPU-baseline leg runs the oracle's own functions on token
    shards: its bytes must equal the single-threaded run's, and a planted
    difference in the reference must be reported."""
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    y = workloads.expert_outputs(wl, N)
    _, n, ref = bench.cpu_baseline(wl, idx, w, x, y, 1)
    assert n == N
    for threads in (1, 3, 7):
        sec, same = bench.cpu_baseline_threaded(wl, idx, w, x, y, 1, threads, ref)
        assert same and sec > 0, threads
    ref["out"][wl.T // 2, 3] ^= 1
    assert not bench.cpu_baseline_threaded(wl, idx, w, x, y, 1, 3, ref)[1]


def test_cold_record_fields():
    wl = workloads.config("v3")
    bc = bench.byte_counts(wl, wl.T * wl.K)
    rec = bench.cold_record(bc, bc["dispatch_logical"] + bc["combine_logical"], [300.0] * 10,
                            [100.0] * 10, [180.0] * 10, "dispatch_fp8_kernel")
    assert rec["step_us"]["median"] == 300.0
    assert rec["roofline"]["combine"]["frac"] == round(bc["combine_alg"] / 180e-6 / 1e9 / 8000, 4)
    assert rec["roofline"]["dispatch"]["kernel"] == "dispatch_fp8_kernel"
    assert rec["value"] == round((bc["dispatch_logical"] + bc["combine_logical"]) / 300e-6 / 1e9, 2)


def test_launch_events_sample_about_twenty_timed_steps():
    """Every timed step runs the whole path; events bracket the dominant
    kernel in every stride-th step, at least once and every step up to 20."""
    for steps in (1, 5, 20, 39):
        assert bench.event_stride(steps) == 1
    assert bench.event_stride(100) == 5
    assert bench.event_stride(1000) == 50
    for steps in (1, 7, 20, 21, 100, 333, 1000):
        s = bench.event_stride(steps)
        sampled = len(range(0, steps, s))
        assert 1 <= sampled and (sampled >= 20 or sampled == steps)


def test_default_step_counts_follow_the_launch_bound_rule():
    """At least 1000 timed steps where a step is tens of microseconds, 100
    for the bandwidth-bound shapes."""
    assert bench.default_steps("tiny") == 1000 and bench.default_steps("decode") == 1000
    for name in ("v3", "skewed", "large"):
        assert bench.default_steps(name) == 100


@pytest.mark.parametrize("name", ["tiny", "decode"])
def test_oracle_timings_beside_the_side_figures(name):
    """The CPU-baseline leg times the oracle on each side figure's inputs:
    the backward calls always, the GEMM-facing dispatches and the
    expert-parallel flow in FP8 mode."""
    wl = workloads.config(name)
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    y = workloads.expert_outputs(wl, N)
    _, _, ref = bench.cpu_baseline(wl, idx, w, x, y, 1)
    side = bench.cpu_side_figures(wl, idx, w, x, y, ref)
    assert set(side["backward"]) >= {"dispatch_backward", "combine_backward_with_grad_w"}
    if wl.use_fp8:
        assert "dispatch_backward_fp8" in side["backward"]
        assert set(side["gemm_layout"]) == {"aligned128_layout_and_dispatch", "fp8_input_dispatch"}
        assert "whole_flow" in side["ep_rank_share"]
    else:
        assert set(side) == {"backward"}
    assert all(v >= 0 for d in side.values() for v in d.values())
    assert bench.cpu_decode_figure() > 0


def test_the_roofline_names_the_combine_form_the_launcher_picks():
    """bench.py names the dominant combine by the library's own rule: outputs
    past the streaming-store threshold run the token-owner form (the large
    workload), smaller ones the segmented form (V3); the threshold is the one
    combine.hip compiles with."""
    import re
    src = open(os.path.join(ROOT, "combine_get_dispatch_scan_amd", "csrc", "combine.hip")).read()
    m = re.search(r"#define EP_COMBINE_STREAM_OUT_BYTES \((\d+)ll << (\d+)\)", src)
    assert m, "threshold define not found"
    assert bench.COMBINE_OWNER_OUT_BYTES == int(m.group(1)) << int(m.group(2))
    v3, large = workloads.config("v3"), workloads.config("large")
    assert v3.T * v3.H * 2 <= bench.COMBINE_OWNER_OUT_BYTES < large.T * large.H * 2
    assert "combine_owner_kernel" in bench.KERNEL_SOURCES
