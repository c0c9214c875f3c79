"""Benchmark: MoE dispatch + combine on one MI355X.

One step runs the whole path once on resident synthetic inputs:
    ep_get_dispatch_layout -> ep_dispatch (FP8) -> ep_handle_recv_counts_async
    -> ep_combine, then the host waits for the counts (an event after the
    readback) and decodes them while combine is still running.
`value` is logical GB/s over the step: the pages count every delivered payload
byte, local traffic included (GeekNews, "Kết quả đo hiệu năng"), so
    dispatch bytes = N * (H * b + 4 * H / 128 [FP8 scales]),  b = 1 (FP8) or 2 (BF16)
    combine bytes  = N * H * 2
with N the number of dispatched (token, k) pairs.

Prints one JSON line.  Default workload: the V3 shape (8192 tokens, hidden
7168, 256 experts, top-8, FP8 dispatch, BF16 combine).
"""
from __future__ import annotations

import argparse
import ctypes
import json
import os
import platform
import statistics
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

METRIC = "dispatch & combine logical GB/s on 1 MI355X (8192×7168 top-8); % HBM peak"
HBM_PEAK_GBPS = 8000.0
# output size past which the library's combine runs the token-owner form
# (its streaming-store threshold)
COMBINE_OWNER_OUT_BYTES = 160 << 20

DESCR = {
    "tiny": "tiny: T=128 H=256 E=16 top-2 P=4, softmax routing, BF16 dispatch",
    "decode": "decode: T=128 H=7168 E=256 top-8 P=8, softmax routing, FP8 dispatch, BF16 combine",
    "v3": "v3: T=8192 H=7168 E=256 top-8 P=8, group-limited gating (4 of 8 groups), FP8 dispatch, BF16 combine",
    "skewed": "skewed: T=4096 H=4096 E=64 top-6 P=8, Zipf(1.2) popularity, 5% masked, BF16 dispatch/combine",
    "large": "large: T=16384 H=7168 E=256 top-8 P=16, uniform routing, Dirichlet(1) weights, FP8 dispatch, BF16 combine",
}


# The pages' own figures for DeepEP's dispatch and combine, reported beside
# ours as context: network-bound multi-GPU runs on NVIDIA hardware, logical
# GB/s counting local traffic too, so not a like-for-like comparison.
PAGES_CONTEXT = {
    "note": "the pages' figures for network-bound DeepEP on other hardware; context, not a target",
    "v3_shape_logical_GBps": [
        # GeekNews (vi.news.hada.io), "Kết quả đo hiệu năng"; aikraft.ru, the benchmark table
        {"hardware": "SM100, EP8 over NVLink, 64 SMs", "dispatch": 726, "combine": 740},
        {"hardware": "SM100, EP8 over NVLink, 24 SMs", "dispatch": 643, "combine": 675},
        {"hardware": "SM100, EP 8x2 over CX7 RDMA, 12 SMs", "dispatch": 90, "combine": 91},
        {"hardware": "SM90, EP 8x2 over CX7 RDMA, 12 SMs", "dispatch": 90, "combine": 81},
        {"hardware": "SM90, EP 8x4 over CX7 RDMA, 6-12 SMs", "dispatch": 61, "combine": 61},
    ],
    # devtrends.ru, performance section; stakiran summary, section 2
    "normal_kernels_GBps": {"H800 NVLink": "150-158", "H800 RDMA": "40-50"},
    "decode_low_latency_us": {"hardware": "H800 + CX7 400 Gb InfiniBand, EP8", "dispatch": 77, "combine": 114},
}


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=None,
                    help="timed steps (default: 1000 for the launch-bound tiny and decode shapes, else 100)")
    ap.add_argument("--warmup", type=int, default=10)
    ap.add_argument("--config", default="v3", choices=sorted(DESCR))
    ap.add_argument("--no-cpu-baseline", action="store_true")
    ap.add_argument("--no-ep-share", action="store_true",
                    help="skip the expert-parallel side figure (its pack dispatch shares the main "
                         "dispatch's kernel and grid, so counter runs of the step leave it out)")
    ap.add_argument("--cpu-runs", type=int, default=6,
                    help="oracle runs of the whole step for the CPU baseline (median; about 10 s at v3)")
    ap.add_argument("--low-latency", action="store_true",
                    help="one-launch static-capacity dispatch (T <= 256) instead of layout + dispatch")
    ap.add_argument("--ll-cap", type=int, default=0,
                    help="rows per expert for --low-latency (default: T, so nothing is dropped)")
    args = ap.parse_args()
    if args.steps is None:
        args.steps = default_steps(args.config)
    return args


def default_steps(config):
    """Timed steps when --steps is not given: 1000 for the shapes whose step is
    a few tens of microseconds (tiny, decode), 100 for the others."""
    return 1000 if config in ("tiny", "decode") else 100


def byte_counts(wl, N):
    T, H, K, E, P = wl.T, wl.H, wl.K, wl.E, wl.P
    b = 1 if wl.use_fp8 else 2
    nb = H // 128
    B = (T + 255) // 256
    disp_logical = N * (H * b + (4 * nb if wl.use_fp8 else 0))
    comb_logical = N * H * 2
    # algorithmic HBM bytes of each call (each byte the definition must read or write once)
    layout_alg = T * K * 8 + T * P + T * K * 4 + B * (E + P + 1) * 4 * 2 + (2 * E + P + 8) * 4
    dispatch_alg = (T * H * 2 + disp_logical + T * K * 4 + T * K * 4 * 2 + T * K * 4 + N * 4
                    + (E + 1) * 4 + B * E * 4)
    combine_alg = N * H * 2 + T * H * 2 + T * K * 8
    return dict(dispatch_logical=disp_logical, combine_logical=comb_logical,
                layout_alg=layout_alg, dispatch_alg=dispatch_alg, combine_alg=combine_alg)


KERNEL_SOURCES = {
    "combine_kernel": ["combine_get_dispatch_scan_amd/csrc/combine.hip",
                       "combine_get_dispatch_scan_amd/csrc/device.h"],
    "combine_owner_kernel": ["combine_get_dispatch_scan_amd/csrc/combine.hip",
                             "combine_get_dispatch_scan_amd/csrc/device.h"],
    "dispatch_fp8_kernel": ["combine_get_dispatch_scan_amd/csrc/dispatch.hip",
                            "combine_get_dispatch_scan_amd/csrc/dispatch_rows.h",
                            "combine_get_dispatch_scan_amd/csrc/device.h"],
    "low_latency_dispatch_kernel": ["combine_get_dispatch_scan_amd/csrc/low_latency.hip",
                                    "combine_get_dispatch_scan_amd/csrc/dispatch_rows.h",
                                    "combine_get_dispatch_scan_amd/csrc/device.h"],
}


def measured_traffic(config, kernel):
    """HBM bytes per launch of `kernel` from the committed rocprofv3 counter
    summary (profiles/<config>_hbm_traffic.md), or None when there is none or
    the kernel's sources changed since the counters were taken."""
    import hashlib
    path = os.path.join(ROOT, "profiles", f"{config}_hbm_traffic.md")
    if not os.path.exists(path) or kernel not in KERNEL_SOURCES:
        return None
    text = open(path).read()
    try:
        blob = text.split("```json", 1)[1].split("```", 1)[0]
        rec = json.loads(blob)[kernel]
    except (IndexError, KeyError, ValueError):
        return None
    h = hashlib.sha256()
    for f in KERNEL_SOURCES[kernel]:
        h.update(open(os.path.join(ROOT, f), "rb").read())
    if h.hexdigest()[:16] != rec["source_sha"]:
        return None
    return int(rec["traffic_bytes"])


def cpu_baseline(wl, idx, w, x, y, runs):
    """The oracle, single-threaded, on the full workload: one whole step per
    run.  Returns the median time, N, and the last run's results (every
    intermediate plus the combine output) for the parity check."""
    import oracle
    times = []
    for _ in range(runs):
        t0 = time.perf_counter()
        r = oracle.run_all(idx, w, x, wl.E, wl.P, wl.use_fp8)
        out = oracle.combine(y, r["slot"], w)
        times.append(time.perf_counter() - t0)
    r["out"] = out
    return statistics.median(times), r["N"], r


def cpu_side_figures(wl, idx, w, x, y, ref):
    """Part of the CPU-baseline leg: the oracle, single thread, one run per
    call, on the inputs of the side figures (ref: the oracle's run of the
    step, slots and combine output included).  Seconds per call."""
    import oracle
    T, K = idx.shape
    H = x.shape[1]
    slot = ref["slot"]

    def secs(fn):
        t0 = time.perf_counter()
        fn()
        return round(time.perf_counter() - t0, 3)
    res = {"backward": {"dispatch_backward": secs(lambda: oracle.dispatch_backward(y, slot)),
                        "combine_backward_with_grad_w":
                            secs(lambda: oracle.combine_backward(ref["out"], y, slot, w, T * K))}}
    if wl.use_fp8:
        res["backward"]["dispatch_backward_fp8"] = secs(
            lambda: oracle.combine_fp8(ref["recv_x"], ref["recv_scales"], slot, None))
        xq = np.random.default_rng(1).integers(0, 256, (T, H), dtype=np.uint8)
        xs = np.ones((T, H // 128), np.float32)
        res["gemm_layout"] = {
            "aligned128_layout_and_dispatch": secs(lambda: oracle.run_all(idx, w, x, wl.E, wl.P, True, align=128)),
            "fp8_input_dispatch": secs(lambda: oracle.dispatch_fp8_input(xq, xs, slot, ref["rows"]))}
        # the expert-parallel flow: one untimed run sizes the expert outputs
        sizing = oracle.ep_one_source(idx, w, x, wl.E, wl.P, True)
        y_parts = [np.zeros((d["unpack"]["rows"], H), np.uint16) + np.uint16(0x3F80)
                   for d in sizing["dest"]]
        res["ep_rank_share"] = {"whole_flow": secs(
            lambda: oracle.ep_one_source(idx, w, x, wl.E, wl.P, True, y_parts=y_parts))}
    return res


def cpu_decode_figure():
    """Part of the CPU-baseline leg: the oracle's one-launch-equivalent
    decode step (static-capacity layout, slots and FP8 rows, then combine),
    single thread, at the decode shape with cap = T rows per expert."""
    import oracle
    import workloads
    wl = workloads.config("decode")
    idx, w, x = workloads.make(wl)
    y = workloads.expert_outputs(wl, wl.E * wl.T)
    t0 = time.perf_counter()
    r = oracle.run_low_latency(idx, w, x, wl.E, wl.P, wl.use_fp8, wl.T)
    oracle.combine(y, r["slot"], w)
    return round(time.perf_counter() - t0, 4)


def cpu_model():
    """The host CPU's model name, read at run time."""
    try:
        with open("/proc/cpuinfo") as f:
            for line in f:
                if line.startswith("model name"):
                    return line.split(":", 1)[1].strip()
    except OSError:
        pass
    return platform.processor() or platform.machine()


def host_threads():
    """Host threads for the threaded oracle leg: the CPUs this process may
    run on, at most 16 (one GPU's share of the host)."""
    try:
        n = len(os.sched_getaffinity(0))
    except AttributeError:
        n = os.cpu_count() or 1
    return max(1, min(16, n))


def cpu_baseline_threaded(wl, idx, w, x, y, runs, threads, ref):
    """The same oracle functions, unchanged, on token shards in `threads`
    host threads (ctypes releases the GIL for each call).  Layout and slots
    stay one sequential pass -- the slot of a pair is a running count over
    all earlier tokens -- and the per-token row work (dispatch rows, then
    combine) is split into contiguous token ranges that write disjoint
    outputs.  Returns the median time and whether every output byte equals
    the single-threaded run's."""
    import ctypes as C
    from concurrent.futures import ThreadPoolExecutor
    import oracle
    L = oracle.lib()
    T, H, K = wl.T, wl.H, wl.K
    nb = H // 128
    p = lambda a, off=0: C.c_void_p(a.ctypes.data + off)
    bounds = [(T * i // threads, T * (i + 1) // threads) for i in range(threads)]
    times = []
    with ThreadPoolExecutor(threads) as pool:
        for _ in range(runs):
            t0 = time.perf_counter()
            r = oracle.run_all(idx, w, None, wl.E, wl.P, wl.use_fp8)
            slot = np.ascontiguousarray(r["slot"], np.int32)
            rows = r["rows"]
            recv = np.zeros((rows, H), np.uint8 if wl.use_fp8 else np.uint16)
            scales = np.zeros((rows, nb), np.float32) if wl.use_fp8 else None
            out = np.empty((T, H), np.uint16)

            def disp(b):
                a, e = b
                L.oracle_dispatch(p(x, a * H * 2), e - a, H, K, p(slot, a * K * 4), int(wl.use_fp8),
                                  p(recv), None if scales is None else p(scales))

            def comb(b):
                a, e = b
                L.oracle_combine(p(y), e - a, H, K, p(slot, a * K * 4), p(w, a * K * 4),
                                 p(out, a * H * 2))
            list(pool.map(disp, bounds))
            list(pool.map(comb, bounds))
            times.append(time.perf_counter() - t0)
    same = (np.array_equal(recv, ref["recv_x"]) and np.array_equal(out, ref["out"]) and
            (scales is None or np.array_equal(scales.view(np.uint32), ref["recv_scales"].view(np.uint32))))
    return statistics.median(times), same


def bf16_ulp_distance(a, b):
    """Largest distance in BF16 ulps between two arrays of BF16 bit patterns
    (an order-preserving map of the patterns to integers; +0 and -0 meet)."""
    def order(v):
        v = v.astype(np.int64)
        return np.where(v >= 0x8000, 0x10000 - v, v + 0x8000)
    return int(np.abs(order(a) - order(b)).max()) if a.size else 0


def parity_verdict(gpu, ref, N, use_fp8):
    """Compare the last timed step's outputs with the oracle's, element by
    element: layout, slots, received rows and scales bit for bit, combine as
    the largest BF16 ulp distance (the bar is 1; same fma order gives 0)."""
    eq = lambda a, b: bool(np.array_equal(a, b))
    v = {
        "layout": eq(gpu["ntpe"], ref["num_tokens_per_expert"]) and eq(gpu["ntpp"], ref["num_tokens_per_partition"])
        and eq(gpu["itip"], ref["is_token_in_partition"]) and gpu["ninv"] == ref["num_invalid"],
        "slot": eq(gpu["slot"], ref["slot"]),
        "recv_rows": eq(gpu["recv"], ref["recv_x"][:N]),
    }
    if use_fp8:
        v["recv_scales"] = eq(gpu["scales"].view(np.uint32), ref["recv_scales"][:N].view(np.uint32))
    ulp = bf16_ulp_distance(gpu["out"], ref["out"])
    verdict = {k: "bit-exact" if ok else "MISMATCH" for k, ok in v.items()}
    verdict["combine_max_ulp"] = ulp
    verdict["combine"] = "bit-exact" if ulp == 0 else ("within 1 ulp" if ulp <= 1 else "MISMATCH")
    verdict["checked"] = "last timed step against the oracle on the full workload"
    return verdict


def measure_ep_share(wl, t_idx, t_w, t_x, time_call):
    """Expert parallelism over P ranks, one rank's share at this workload's
    shape, each call timed alone (events, 10 launches, mean).  The sender
    packs its tokens per destination; the P packed blocks, whose local ids are
    valid for any one rank's E/P experts, stand in for the rows one rank
    receives from P sources (the exchange itself is not on one GPU)."""
    import torch
    import combine_get_dispatch_scan_amd as ep
    T, H, K, E, P = wl.T, wl.H, wl.K, wl.E, wl.P
    Kp, epp, nb = min(K, P), E // P, H // 128
    dev = t_x.device
    sp = ep._stream()
    p = lambda t: None if t is None else t.data_ptr()

    def ok(rc):
        if rc != 0:
            raise RuntimeError(ep.ep_last_error())
    part = torch.empty((T, Kp), dtype=torch.int64, device=dev)
    route = lambda: ok(ep.ep_rank_routing(p(t_idx), T, K, E, P, p(part), sp))
    route()
    lay = ep.get_dispatch_layout(part, P, P)
    hp = lay.handle.c
    cap = T * Kp
    send = torch.empty((cap, H), dtype=torch.uint8, device=dev)
    send_sc = torch.empty((cap, nb), dtype=torch.float32, device=dev)
    li = torch.full((cap, K), -1, dtype=torch.int64, device=dev)
    lw = torch.zeros((cap, K), dtype=torch.float32, device=dev)
    pack_layout = lambda: ok(ep.ep_get_dispatch_layout(p(part), T, Kp, P, P, p(lay.num_tokens_per_partition),
                                                       p(lay.num_tokens_per_expert), p(lay.is_token_in_partition),
                                                       p(lay.num_invalid), p(lay.handle.ws),
                                                       lay.handle.ws.numel(), hp, sp))
    pack = lambda: ok(ep.ep_dispatch(p(t_x), None, H, 1, p(send), p(send_sc), cap, hp, sp))
    pack()
    meta = lambda: ok(ep.ep_pack_metadata(p(t_idx), p(t_w), K, E, p(part), hp, p(li), p(lw), sp))
    meta()
    _, R, _ = ep.handle_recv_counts(lay.handle)
    # the receiver: all R packed rows as one rank's receive buffer
    lay_r = ep.get_dispatch_layout(li[:R], epp, 1)
    hr = lay_r.handle.c
    capr = R * K
    recv = torch.empty((capr, H), dtype=torch.uint8, device=dev)
    recv_sc = torch.empty((capr, nb), dtype=torch.float32, device=dev)
    unpack_layout = lambda: ok(ep.ep_get_dispatch_layout(p(li), R, K, epp, 1, p(lay_r.num_tokens_per_partition),
                                                         p(lay_r.num_tokens_per_expert),
                                                         p(lay_r.is_token_in_partition), p(lay_r.num_invalid),
                                                         p(lay_r.handle.ws), lay_r.handle.ws.numel(), hr, sp))
    unpack = lambda: ok(ep.ep_dispatch_ex(p(send), p(send_sc), p(lw), H, 1, 0, p(recv), p(recv_sc), capr, hr, sp))
    unpack()
    _, Nr, _ = ep.handle_recv_counts(lay_r.handle)
    y = torch.randn((max(Nr, 1), H), device=dev).to(torch.bfloat16)
    partial = torch.empty((max(R, 1), H), dtype=torch.bfloat16, device=dev)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    reduce_ = lambda: ok(ep.ep_combine(p(y), hr, None, p(partial), sp))
    origin = lambda: ok(ep.ep_dispatch_backward(p(partial), hp, p(out), sp))
    B, Br = (T + 255) // 256, (R + 255) // 256
    calls = {
        "rank_routing": (route, T * K * 8 + T * Kp * 8),
        "pack_layout": (pack_layout, T * Kp * 12 + T * P + B * (2 * P + 1) * 4 * 2),
        "pack_dispatch": (pack, T * H * 2 + R * (H + 4 * nb) + T * Kp * 16 + R * 4),
        "pack_metadata": (meta, T * Kp * 12 + T * K * 12 + R * K * 12),
        "unpack_layout": (unpack_layout, R * K * 12 + R + Br * (2 * epp + 2) * 4 * 2),
        "unpack_dispatch": (unpack, R * (H + 4 * nb) + Nr * (H + 4 * nb) + R * K * 16 + Nr * 4),
        "expert_prereduce": (reduce_, Nr * H * 2 + R * H * 2 + R * K * 8),
        "origin_sum": (origin, R * H * 2 + T * H * 2 + T * Kp * 4),
    }
    res = {"packed_rows": int(R), "received_pairs": int(Nr),
           "note": "one rank's share; the P packed blocks stand in for the rows received from P sources"}
    total = 0.0
    for name, (fn, nbytes) in calls.items():
        ms = time_call(fn)
        total += ms
        res[name] = {"us": round(ms * 1e3, 2), "hbm_frac": round(nbytes / (ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)}
    res["total_us"] = round(total * 1e3, 2)
    return res


def event_stride(steps):
    """Every how many timed steps the dominant kernel is bracketed by events:
    about 20 sampled launches, every step when there are 20 or fewer."""
    return max(1, steps // 20)


def cold_record(bc, logical, step_us, disp_us, comb_us, disp_kernel, comb_kernel="combine_kernel"):
    """Cold-cache figures: every measured step or call runs right after a
    2 GiB read that evicts the Infinity Cache and the L2s; medians of 10."""
    med = lambda v: v[len(v) // 2]
    frac = lambda nbytes, us: round(nbytes / (us * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4)
    return {
        "value": round(logical / (med(step_us) * 1e-6) / 1e9, 2), "unit": "GB/s",
        "protocol": "each step (or call) after reading a 2 GiB scratch buffer; two events around it; "
                    "median of 10",
        "step_us": {"median": round(med(step_us), 2), "min": round(step_us[0], 2)},
        "roofline": {
            "dispatch": {"kernel": disp_kernel,
                         "us": round(med(disp_us), 2), "bytes_per_launch": bc["dispatch_alg"],
                         "frac": frac(bc["dispatch_alg"], med(disp_us))},
            "combine": {"kernel": comb_kernel, "us": round(med(comb_us), 2),
                        "bytes_per_launch": bc["combine_alg"], "frac": frac(bc["combine_alg"], med(comb_us))},
            "peak": HBM_PEAK_GBPS, "unit": "GB/s", "bound": "hbm",
        },
        "hbm_frac_step": round((bc["layout_alg"] + bc["dispatch_alg"] + bc["combine_alg"]) /
                               (med(step_us) * 1e-6) / 1e9 / HBM_PEAK_GBPS, 4),
    }


def bench_low_latency(args):
    wl_T = __import__("workloads").config(args.config).T
    if wl_T > 256:
        print(f"--low-latency takes at most 256 tokens ({args.config} has {wl_T})", file=sys.stderr)
        sys.exit(2)
    print(json.dumps(measure_low_latency(args.config, args.ll_cap, args.steps, args.warmup)), flush=True)


def measure_low_latency(config, ll_cap, steps, warmup):
    """Decode step through the one-launch dispatch: ep_low_latency_dispatch ->
    counts readback -> ep_combine, timed eagerly and as a replayed HIP graph
    (dispatch + combine captured once).  Returns the JSON record."""
    import torch
    import combine_get_dispatch_scan_amd as ep
    import workloads

    ep.load()
    dev = torch.device("cuda:0")
    wl = workloads.config(config)
    T, H, K, E, P = wl.T, wl.H, wl.K, wl.E, wl.P
    cap = ll_cap or T
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    y = workloads.expert_outputs(wl, E * cap)
    t_idx = torch.from_numpy(idx).to(dev)
    t_w = torch.from_numpy(w).to(dev)
    t_x = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    t_y = torch.from_numpy(y.view(np.int16)).to(dev).view(torch.bfloat16)
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    host_buf = torch.empty(E + 5, dtype=torch.int32, pin_memory=True)
    counts = (ctypes.c_int32 * E)()
    nrecv = ctypes.c_int32(0)
    counts_ready = torch.cuda.Event()
    recv, sc, lay = ep.low_latency_dispatch(t_x, t_idx, t_w, E, P, cap, wl.use_fp8)
    h = lay.handle.c
    ws = lay.handle.ws
    stream = torch.cuda.current_stream()
    sp = ep._stream()
    p = lambda t: None if t is None else t.data_ptr()
    mean = lambda v: sum(v) / len(v)
    ll_args = (p(t_x), p(t_idx), p(t_w), T, H, K, E, P, int(wl.use_fp8), cap, p(recv), p(sc),
               p(lay.num_tokens_per_partition), p(lay.num_tokens_per_expert),
               p(lay.is_token_in_partition), p(lay.num_invalid), p(ws), ws.numel(), h, sp)

    def fwd():
        s_now = ep._stream()          # the capture stream under graph capture
        rc = ep.ep_low_latency_dispatch(*ll_args[:-1], s_now)
        rc |= ep.ep_combine(p(t_y), h, None, p(out), s_now)
        if rc != 0:
            raise RuntimeError(ep.ep_last_error())

    def step():
        rc = ep.ep_low_latency_dispatch(*ll_args)
        rc |= ep.ep_handle_recv_counts_async(h, host_buf.data_ptr(), sp)
        counts_ready.record(stream)
        rc |= ep.ep_combine(p(t_y), h, None, p(out), sp)
        # the grouped GEMM would need the counts here; combine is already queued
        counts_ready.synchronize()
        rc |= ep.ep_recv_counts_decode(h, host_buf.data_ptr(), counts, ctypes.byref(nrecv))
        if rc != 0:
            raise RuntimeError(ep.ep_last_error())

    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    assert nrecv.value == N, (nrecv.value, N)
    torch.cuda.synchronize()
    stamps = [time.perf_counter()]
    for i in range(steps):
        step()
        stamps.append(time.perf_counter())
    torch.cuda.synchronize()
    ms_per_step = (time.perf_counter() - stamps[0]) * 1e3 / steps
    # each step ends when the host holds the counts (combine still queued), so
    # the intervals between step ends spread around the step time; a step the
    # host reached late is followed by a short interval, so no minimum
    per_step_us = sorted((b - a) * 1e6 for a, b in zip(stamps, stamps[1:]))
    step_stats = {"median": round(statistics.median(per_step_us), 2),
                  "p90": round(per_step_us[int(0.9 * (len(per_step_us) - 1))], 2),
                  "note": "intervals between the host's step ends"}

    # kernel duration: back-to-back launches keep the GPU busy, so events
    # around a batch time the kernels rather than the host's launch gaps
    def batch_us(fn, n=200):
        fn()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(n):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) * 1e3 / n
    disp_us = batch_us(lambda: ep.ep_low_latency_dispatch(*ll_args))
    comb_us = batch_us(lambda: ep.ep_combine(p(t_y), h, None, p(out), sp))
    disp_ms = disp_us * 1e-3
    # a plain 1 GiB copy and fill in the same run (the counters' calibration)
    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy_gbps = (2 << 30) / (batch_us(lambda: dst.copy_(src), 5) * 1e-6) / 1e9
    fill_gbps = (1 << 30) / (batch_us(lambda: dst.fill_(3), 5) * 1e-6) / 1e9
    del src, dst
    # floors at this size, timed like the dispatch: each call launched 50
    # times inside one captured HIP graph (no host work between launches),
    # per-launch time from two events around a replay.  A fill of 4 bytes
    # is launch and completion alone; a fill of as many bytes as the
    # dispatch writes adds the writes.  int32 fills are kernels (no memset
    # node in the graph).
    def graph_us(fn, n=50):
        side_s = torch.cuda.Stream()
        side_s.wait_stream(stream)
        with torch.cuda.stream(side_s):
            fn()
        stream.wait_stream(side_s)
        torch.cuda.synchronize()
        gr = torch.cuda.CUDAGraph()
        with torch.cuda.graph(gr):
            for _ in range(n):
                fn()
        gr.replay()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        gr.replay()
        a1.record(stream)
        torch.cuda.synchronize()
        return a0.elapsed_time(a1) * 1e3 / n
    b_row = 1 if wl.use_fp8 else 2
    written = N * (H * b_row + (4 * (H // 128) if wl.use_fp8 else 0)) + T * K * 8 + T * P
    wbuf = torch.empty((written + 3) // 4, dtype=torch.int32, device=dev)
    tiny = torch.empty(1, dtype=torch.int32, device=dev)

    def ll_only():
        if ep.ep_low_latency_dispatch(*ll_args[:-1], ep._stream()):
            raise RuntimeError(ep.ep_last_error())
    floors = {"protocol": "50 launches in one captured graph, per launch",
              "low_latency_dispatch": round(graph_us(ll_only), 2),
              "fill_of_the_written_bytes": round(graph_us(lambda: wbuf.fill_(7)), 2),
              "fill_of_4_bytes": round(graph_us(lambda: tiny.fill_(7)), 2),
              "written_bytes": written}
    del wbuf, tiny

    # the same forward captured once and replayed (no host work per step)
    side = torch.cuda.Stream()
    side.wait_stream(stream)
    with torch.cuda.stream(side):
        fwd()
    stream.wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fwd()
    for _ in range(warmup):
        g.replay()
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(steps):
        g.replay()
    torch.cuda.synchronize()
    graph_ms = (time.perf_counter() - t0) * 1e3 / steps
    print(f"[bench] low-latency {config}: {ms_per_step * 1e3:.1f} us/step eager, "
          f"{graph_ms * 1e3:.1f} us/step graph, kernels: dispatch {disp_us:.2f} us, "
          f"combine {comb_us:.2f} us",
          file=sys.stderr, flush=True)

    b = 1 if wl.use_fp8 else 2
    nb = H // 128
    disp_logical = N * (H * b + (4 * nb if wl.use_fp8 else 0))
    comb_logical = N * H * 2
    # ids and weights read, slots + weight copy + mask + counts written, x read once, rows written
    disp_alg = (T * K * 8 + T * K * 4 + T * K * 8 + T * P + (2 * E + P + 8) * 4 + T * H * 2
                + disp_logical)
    disp_gbps = disp_alg / (disp_ms * 1e-3) / 1e9
    value = (disp_logical + comb_logical) / (ms_per_step * 1e-3) / 1e9
    res = {
        "metric": "low-latency dispatch & combine logical GB/s on 1 MI355X",
        "value": round(value, 2), "unit": "GB/s", "n_gpus": 1, "steps": steps,
        "warmup": warmup, "ms_per_step": round(ms_per_step, 5), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None,
        "dtype": "fp8e4m3+bf16/fp32-acc" if wl.use_fp8 else "bf16/fp32-acc", "data": "synthetic",
        "config": {"workload": DESCR[config] + ", one-launch static-capacity dispatch",
                   "tokens": T, "hidden": H, "experts": E, "topk": K, "partitions": P,
                   "dispatched_pairs": N, "rows_per_expert": cap},
        "us_per_step_stats": step_stats,
        "graph_replay_us_per_step": round(graph_ms * 1e3, 2),
        "kernels_us": {"low_latency_dispatch": round(disp_us, 2), "combine": round(comb_us, 2)},
        "ceilings_GBps": {"torch_copy_1GiB": round(copy_gbps, 1), "torch_fill_1GiB": round(fill_gbps, 1)},
        "latency_floors_us": floors,
        "roofline": {"bound": "hbm", "kernel": "low_latency_dispatch_kernel",
                     "achieved": round(disp_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
                     "frac": round(disp_gbps / HBM_PEAK_GBPS, 4), "bytes_per_launch": disp_alg,
                     "avg_launch_us": round(disp_ms * 1e3, 2),
                     "traffic": measured_traffic(f"{config}_low_latency", "low_latency_dispatch_kernel")},
    }
    return res


def main():
    args = parse()
    world = int(os.environ.get("WORLD_SIZE", "1"))
    if args.gpus != 1 or world != 1:
        print(f"bench.py measures one GPU only (asked for --gpus {args.gpus}, WORLD_SIZE={world}); "
              "the path runs on one MI355X and is not sharded across GPUs.", file=sys.stderr)
        sys.exit(2)
    if args.low_latency:
        return bench_low_latency(args)

    import torch
    import combine_get_dispatch_scan_amd as ep
    import workloads

    ep.load()
    dev = torch.device("cuda:0")
    wl = workloads.config(args.config)
    print(f"[bench] generating {args.config}", file=sys.stderr, flush=True)
    idx, w, x = workloads.make(wl)
    N = int((idx >= 0).sum())
    y = workloads.expert_outputs(wl, N)
    T, H, K, E, P = wl.T, wl.H, wl.K, wl.E, wl.P
    cap = T * K

    t_idx = torch.from_numpy(idx).to(dev)
    t_w = torch.from_numpy(w).to(dev)
    t_x = torch.from_numpy(x.view(np.int16)).to(dev).view(torch.bfloat16)
    t_y = torch.from_numpy(y.view(np.int16)).to(dev).view(torch.bfloat16)
    ws = torch.empty(ep.ep_workspace_bytes(T, K, E, P), dtype=torch.uint8, device=dev)
    ntpp = torch.empty(P, dtype=torch.int32, device=dev)
    ntpe = torch.empty(E, dtype=torch.int32, device=dev)
    itip = torch.empty((T, P), dtype=torch.uint8, device=dev)
    ninv = torch.empty(1, dtype=torch.int32, device=dev)
    if wl.use_fp8:
        recv = torch.empty((cap, H), dtype=torch.uint8, device=dev)
        scales = torch.empty((cap, H // 128), dtype=torch.float32, device=dev)
    else:
        recv = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
        scales = None
    out = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    counts = (ctypes.c_int32 * E)()
    nrecv = ctypes.c_int32(0)
    host_buf = torch.empty(E + 5, dtype=torch.int32, pin_memory=True)
    counts_ready = torch.cuda.Event()
    h = ep.ep_handle_t()
    stream = torch.cuda.current_stream()
    sp = ep._stream()
    p = lambda t: None if t is None else t.data_ptr()

    def step(ev=None, dom=None):
        """One pass of the path.  ev: 4 events around the three calls, or
        (with dom) 2 events around the dominant call only, or (dom "all") 2
        events around the whole step."""
        if ev is not None and dom in (None, "all"):
            ev[0].record(stream)
        rc = ep.ep_get_dispatch_layout(p(t_idx), T, K, E, P, p(ntpp), p(ntpe), p(itip), p(ninv),
                                       p(ws), ws.numel(), h, sp)
        if ev is not None and dom is None:
            ev[1].record(stream)
        if dom == "dispatch":
            ev[0].record(stream)
        rc |= ep.ep_dispatch(p(t_x), p(t_w), H, int(wl.use_fp8), p(recv), p(scales), cap, h, sp)
        if dom == "dispatch":
            ev[1].record(stream)
        rc |= ep.ep_handle_recv_counts_async(h, host_buf.data_ptr(), sp)
        counts_ready.record(stream)
        if ev is not None and dom is None:
            ev[2].record(stream)
        if dom == "combine":
            ev[0].record(stream)
        rc |= ep.ep_combine(p(t_y), h, None, p(out), sp)
        if dom == "combine":
            ev[1].record(stream)
        if ev is not None and dom is None:
            ev[3].record(stream)
        if dom == "all":
            ev[1].record(stream)
        # the grouped GEMM would need the counts here; combine is already queued
        counts_ready.synchronize()
        rc |= ep.ep_recv_counts_decode(h, host_buf.data_ptr(), counts, ctypes.byref(nrecv))
        if rc != 0:
            raise RuntimeError(f"step failed: {ep.ep_last_error()}")

    print(f"[bench] warmup {args.warmup}", file=sys.stderr, flush=True)
    for _ in range(args.warmup):
        step()
    torch.cuda.synchronize()
    assert nrecv.value == N, (nrecv.value, N)

    # phase breakdown (untimed): events around every call
    n_ph = max(5, min(args.steps, 20))
    evs = [[torch.cuda.Event(enable_timing=True) for _ in range(4)] for _ in range(n_ph)]
    for i in range(n_ph):
        step(evs[i])
    torch.cuda.synchronize()
    mean = lambda v: sum(v) / len(v)
    # (the dispatch phase includes the enqueue of the count readback)
    phases = {"layout": mean([e[0].elapsed_time(e[1]) for e in evs]),
              "dispatch": mean([e[1].elapsed_time(e[2]) for e in evs]),
              "combine": mean([e[2].elapsed_time(e[3]) for e in evs])}
    # dominant kernel: the larger of dispatch and combine (one kernel launch each)
    dom = max(("dispatch", "combine"), key=lambda k: phases[k])

    # timed region: exactly K steps, wall clock, synchronised on both sides.
    # Two events bracket the dominant kernel on the launch stream in every
    # stride-th step (about 20 launches sampled); each bracketed step carries
    # about 7 us of GPU idle for its two timing markers, so bracketing every
    # step would add that to every step's time
    stride = event_stride(args.steps)
    dev_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)]
              for _ in range(0, args.steps, stride)]
    torch.cuda.synchronize()
    t0 = time.perf_counter()
    stamps = [t0]
    for i in range(args.steps):
        if i % stride == 0:
            step(dev_ev[i // stride], dom)
        else:
            step()
        stamps.append(time.perf_counter())
    torch.cuda.synchronize()
    t1 = time.perf_counter()
    ms_per_step = (t1 - t0) * 1e3 / args.steps
    # each step ends when the host holds the counts (combine still queued), so
    # the intervals between step ends spread around the step time; a step the
    # host reached late is followed by a short interval, so no minimum
    per_step_us = sorted((b - a) * 1e6 for a, b in zip(stamps, stamps[1:]))
    step_stats = {"median": round(statistics.median(per_step_us), 2),
                  "p90": round(per_step_us[int(0.9 * (len(per_step_us) - 1))], 2),
                  "note": "intervals between the host's step ends"}
    dom_all = sorted(e[0].elapsed_time(e[1]) for e in dev_ev)
    dom_ms = mean(dom_all)
    dom_stats = {"median": round(dom_all[len(dom_all) // 2] * 1e3, 2), "min": round(dom_all[0] * 1e3, 2),
                 "p90": round(dom_all[min(len(dom_all) - 1, int(0.9 * len(dom_all)))] * 1e3, 2)}
    print(f"[bench] timed {args.steps} steps: {ms_per_step:.4f} ms/step, {dom} {dom_ms * 1e3:.2f} us",
          file=sys.stderr, flush=True)
    # the last timed step's outputs, kept for the parity check against the
    # oracle that the CPU-baseline leg runs on the same inputs
    gpu_out = None
    if not args.no_cpu_baseline:
        slot_off = h.slot - ws.data_ptr()
        gpu_out = {
            "ntpe": ntpe.cpu().numpy(), "ntpp": ntpp.cpu().numpy(), "itip": itip.cpu().numpy(),
            "ninv": int(ninv.cpu()[0]),
            "slot": ws[slot_off:slot_off + T * K * 4].view(torch.int32).cpu().numpy().reshape(T, K),
            "recv": (recv[:N].cpu().numpy() if wl.use_fp8
                     else recv[:N].view(torch.int16).cpu().numpy().view(np.uint16)),
            "scales": scales[:N].cpu().numpy() if wl.use_fp8 else None,
            "out": out.view(torch.int16).cpu().numpy().view(np.uint16),
        }

    # cold steps: reading a 2 GiB scratch buffer before each step evicts the
    # Infinity Cache (256 MB) and the L2s with clean lines (a fill would leave
    # dirty ones for the step to write back); two events bracket the step
    scratch = torch.ones(1 << 29, dtype=torch.float32, device=dev)
    cold_ev = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(10)]
    for e in cold_ev:
        scratch.amax()
        step(e, "all")
    torch.cuda.synchronize()
    cold_us = sorted(e[0].elapsed_time(e[1]) * 1e3 for e in cold_ev)

    # cold calls: dispatch and combine each timed alone (two events) right
    # after the same 2 GiB read, so neither finds its inputs in a cache
    def cold_call(fn, reps=10):
        evs_c = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in evs_c:
            scratch.amax()
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return sorted(e[0].elapsed_time(e[1]) * 1e3 for e in evs_c)

    def _disp():
        if ep.ep_dispatch(p(t_x), p(t_w), H, int(wl.use_fp8), p(recv), p(scales), cap, h, sp):
            raise RuntimeError(ep.ep_last_error())

    def _comb():
        if ep.ep_combine(p(t_y), h, None, p(out), sp):
            raise RuntimeError(ep.ep_last_error())
    cold_disp_us = cold_call(_disp)
    cold_comb_us = cold_call(_comb)
    del scratch

    bc = byte_counts(wl, N)
    dom_bytes = bc["dispatch_alg"] if dom == "dispatch" else bc["combine_alg"]
    dom_gbps = dom_bytes / (dom_ms * 1e-3) / 1e9
    # the combine form the launcher picks: the token-owner kernel for outputs
    # past 160 MiB (streaming stores), the segmented kernel below
    combine_name = "combine_owner_kernel" if T * H * 2 > COMBINE_OWNER_OUT_BYTES else "combine_kernel"
    dom_kernel = {"dispatch": "dispatch_fp8_kernel" if wl.use_fp8 else "dispatch_bf16_kernel",
                  "combine": combine_name}[dom]

    # practical ceilings on this GPU, same run: a plain 1 GiB device copy and fill
    def rate(fn, nbytes, reps=10):
        fn()
        torch.cuda.synchronize()
        a0 = torch.cuda.Event(enable_timing=True)
        a1 = torch.cuda.Event(enable_timing=True)
        a0.record(stream)
        for _ in range(reps):
            fn()
        a1.record(stream)
        torch.cuda.synchronize()
        return nbytes * reps / (a0.elapsed_time(a1) * 1e-3) / 1e9
    # backward calls on the same routing (reported beside the forward step):
    # dispatch backward = unit-weight combine of a [rows, H] gradient;
    # combine backward = weight-scaled rows of grad_out plus grad_w dot products
    grad_x = torch.empty((T, H), dtype=torch.bfloat16, device=dev)
    grad_y = torch.empty((cap, H), dtype=torch.bfloat16, device=dev)
    grad_w = torch.empty((T, K), dtype=torch.float32, device=dev)

    def time_call(fn, reps=10):
        fn()
        torch.cuda.synchronize()
        evs_b = [[torch.cuda.Event(enable_timing=True) for _ in range(2)] for _ in range(reps)]
        for e in evs_b:
            e[0].record(stream)
            fn()
            e[1].record(stream)
        torch.cuda.synchronize()
        return mean([e[0].elapsed_time(e[1]) for e in evs_b])

    def _ok(rc):
        if rc != 0:
            raise RuntimeError(ep.ep_last_error())
    db_ms = time_call(lambda: _ok(ep.ep_dispatch_backward(p(t_y), h, p(grad_x), sp)))
    cb_ms = time_call(lambda: _ok(ep.ep_combine_backward(p(out), p(t_y), h, None, p(grad_y),
                                                         p(grad_w), sp)))
    db_bytes = N * H * 2 + T * H * 2 + T * K * 4
    cb_bytes = T * H * 2 + 2 * N * H * 2 + T * K * 12
    backward = {
        "dispatch_backward_us": round(db_ms * 1e3, 2),
        "dispatch_backward_hbm_frac": round(db_bytes / (db_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "combine_backward_us": round(cb_ms * 1e3, 2),
        "combine_backward_hbm_frac": round(cb_bytes / (cb_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
    }
    if wl.use_fp8:
        # the dequantising backward of dispatch, on FP8 rows + scales (here dispatch's own)
        d8_ms = time_call(lambda: _ok(ep.ep_dispatch_backward_fp8(p(recv), p(scales), h, p(grad_x), sp)))
        d8_bytes = N * H + N * (H // 128) * 4 + T * H * 2 + T * K * 4
        backward["dispatch_backward_fp8_us"] = round(d8_ms * 1e3, 2)
        backward["dispatch_backward_fp8_hbm_frac"] = round(d8_bytes / (d8_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4)
    del grad_x, grad_y, grad_w

    # GEMM-facing options on the same routing (reported beside the step):
    # expert blocks aligned to 128 rows with column-major scales, and
    # pre-quantised FP8 input passed through
    gemm = {}
    if wl.use_fp8:
        A = 128
        lay_a = ep.get_dispatch_layout(t_idx, E, P, expert_alignment=A)
        cap_a = T * K + E * (A - 1)
        ld = (cap_a + 3) // 4 * 4
        recv_a = torch.empty((cap_a, H), dtype=torch.uint8, device=dev)
        sc_a = torch.empty((H // 128, ld), dtype=torch.float32, device=dev)
        ha = lay_a.handle.c

        def disp_aligned():
            _ok(ep.ep_dispatch_ex(p(t_x), None, p(t_w), H, 1, ld, p(recv_a), p(sc_a), cap_a, ha, sp))
        al_ms = time_call(disp_aligned)
        cnt_a, rows_a, _ = ep.handle_recv_counts(lay_a.handle)
        pad = rows_a - N
        al_bytes = bc["dispatch_alg"] + pad * (H + (H // 128) * 4)
        xq = torch.randint(0, 256, (T, H), dtype=torch.uint8, device=dev)
        xs = torch.rand((T, H // 128), dtype=torch.float32, device=dev)

        def disp_fp8in():
            _ok(ep.ep_dispatch_ex(p(xq), p(xs), p(t_w), H, 1, 0, p(recv), p(scales), cap, h, sp))
        in_ms = time_call(disp_fp8in)
        in_bytes = bc["dispatch_alg"] - T * H * 2 + T * H + T * (H // 128) * 4
        gemm = {
            "aligned128_colmajor_dispatch_us": round(al_ms * 1e3, 2),
            "aligned128_padding_rows": int(pad),
            "aligned128_hbm_frac": round(al_bytes / (al_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "fp8_input_dispatch_us": round(in_ms * 1e3, 2),
            "fp8_input_hbm_frac": round(in_bytes / (in_ms * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        }
        del recv_a, sc_a, xq, xs, lay_a
        # the timed step's handle must hold the BF16-input dispatch again
        _ok(ep.ep_dispatch(p(t_x), p(t_w), H, 1, p(recv), p(scales), cap, h, sp))

    ep_share = {}
    if wl.use_fp8 and not args.no_ep_share:
        ep_share = measure_ep_share(wl, t_idx, t_w, t_x, time_call)
        # the timed step's handle must hold the plain dispatch again
        _ok(ep.ep_get_dispatch_layout(p(t_idx), T, K, E, P, p(ntpp), p(ntpe), p(itip), p(ninv),
                                      p(ws), ws.numel(), h, sp))
        _ok(ep.ep_dispatch(p(t_x), p(t_w), H, 1, p(recv), p(scales), cap, h, sp))

    src = torch.empty(1 << 30, dtype=torch.uint8, device=dev).fill_(1)
    dst = torch.empty_like(src)
    copy_gbps = rate(lambda: dst.copy_(src), 2 << 30)
    fill_gbps = rate(lambda: dst.fill_(3), 1 << 30)
    del src, dst

    logical = bc["dispatch_logical"] + bc["combine_logical"]
    value = logical / (ms_per_step * 1e-3) / 1e9
    alg_step = bc["layout_alg"] + bc["dispatch_alg"] + bc["combine_alg"]
    res = {
        "metric": METRIC,
        "value": round(value, 2),
        "unit": "GB/s",
        "n_gpus": 1,
        "steps": args.steps,
        "warmup": args.warmup,
        "ms_per_step": round(ms_per_step, 5),
        "higher_is_better": True,
        "scaling": "weak",
        "vs_baseline": None,
        "dtype": "fp8e4m3+bf16/fp32-acc" if wl.use_fp8 else "bf16/fp32-acc",
        "data": "synthetic",
        "config": {"workload": DESCR[args.config], "tokens": T, "hidden": H, "experts": E,
                   "topk": K, "partitions": P, "dispatched_pairs": N,
                   "fp8_dispatch": bool(wl.use_fp8), "capacity_rows": cap},
        "roofline": {
            "bound": "hbm", "kernel": dom_kernel,
            "achieved": round(dom_gbps, 1), "peak": HBM_PEAK_GBPS, "unit": "GB/s",
            "frac": round(dom_gbps / HBM_PEAK_GBPS, 4),
            "bytes_per_launch": dom_bytes, "avg_launch_us": round(dom_ms * 1e3, 2),
            "launch_us": dom_stats,
            "launch_events": f"two events around the kernel in every {stride}th timed step "
                             f"({len(dev_ev)} launches)",
            "traffic": measured_traffic(args.config, dom_kernel),
        },
        "value_protocol": "warm: the K timed steps run back to back on resident inputs, caches not "
                          "flushed (one step touches about 1.6 GB against the 256 MB Infinity Cache)",
        "cold": cold_record(bc, logical, cold_us, cold_disp_us, cold_comb_us,
                            "dispatch_fp8_kernel" if wl.use_fp8 else "dispatch_bf16_kernel", combine_name),
        "step_us": step_stats,
        "phases_us": {k: round(v * 1e3, 2) for k, v in phases.items()},
        "ceilings_GBps": {"torch_copy_1GiB": round(copy_gbps, 1), "torch_fill_1GiB": round(fill_gbps, 1)},
        "backward": backward,
        "gemm_layout": gemm,
        "ep_rank_share": ep_share,
        "logical_GBps": {
            "dispatch": round(bc["dispatch_logical"] / ((phases["layout"] + phases["dispatch"]) * 1e-3) / 1e9, 1),
            "combine": round(bc["combine_logical"] / (phases["combine"] * 1e-3) / 1e9, 1),
        },
        "pages_context": PAGES_CONTEXT,
        "hbm_frac_step": round(alg_step / (ms_per_step * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        "hbm_frac_kernels": {
            "dispatch": round(bc["dispatch_alg"] / (phases["dispatch"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
            "combine": round(bc["combine_alg"] / (phases["combine"] * 1e-3) / 1e9 / HBM_PEAK_GBPS, 4),
        },
    }

    if args.config == "v3":
        # the decode-shape path through the one-launch dispatch, for reference
        ll = measure_low_latency("decode", 0, 1000, 10)
        res["low_latency_decode"] = {
            "workload": ll["config"]["workload"], "steps": ll["steps"],
            "us_per_step": round(ll["ms_per_step"] * 1e3, 2),
            "us_per_step_stats": ll["us_per_step_stats"],
            "graph_replay_us_per_step": ll["graph_replay_us_per_step"], "kernels_us": ll["kernels_us"],
            "dispatch_roofline_frac": ll["roofline"]["frac"], "latency_floors_us": ll["latency_floors_us"]}

    if not args.no_cpu_baseline:
        print(f"[bench] cpu baseline ({args.cpu_runs} oracle runs)", file=sys.stderr, flush=True)
        sec, n_cpu, ref = cpu_baseline(wl, idx, w, x, y, args.cpu_runs)
        assert n_cpu == N
        res["parity"] = parity_verdict(gpu_out, ref, N, wl.use_fp8)
        print(f"[bench] parity: {res['parity']}", file=sys.stderr, flush=True)
        print("[bench] cpu oracle beside the side figures", file=sys.stderr, flush=True)
        side = cpu_side_figures(wl, idx, w, x, y, ref)
        for key, secs_map in side.items():
            if res.get(key):
                res[key]["cpu_oracle_s"] = dict(secs_map, note="the oracle, one thread, one run per call")
        if res.get("low_latency_decode"):
            res["low_latency_decode"]["cpu_oracle_s"] = {"step": cpu_decode_figure(),
                                                         "note": "the oracle, one thread, one run"}
        nthr = host_threads()
        print(f"[bench] cpu baseline, {nthr} threads", file=sys.stderr, flush=True)
        sec_mt, same_mt = cpu_baseline_threaded(wl, idx, w, x, y, args.cpu_runs, nthr, ref)
        res["cpu_baseline"] = {
            "value": round(logical / sec / 1e9, 4), "unit": "GB/s", "cores": 1, "kind": "oracle",
            "sample": f"whole step (layout, slots, {'FP8' if wl.use_fp8 else 'BF16'} dispatch, combine) "
                      f"on the full {args.config} workload, single thread, median of {args.cpu_runs} runs "
                      f"({sec:.2f} s each); host CPU {cpu_model()}, {os.cpu_count()} logical CPUs visible",
            "threaded": {
                "value": round(logical / sec_mt / 1e9, 4), "unit": "GB/s", "cores": nthr,
                "seconds": round(sec_mt, 3), "identical_bytes": bool(same_mt),
                "sample": "the same oracle functions on contiguous token shards in host threads "
                          "(layout and slots one sequential pass); median of "
                          f"{args.cpu_runs} runs, every output byte compared with the single-thread run",
            },
        }
    print(json.dumps(res), flush=True)


if __name__ == "__main__":
    main()
