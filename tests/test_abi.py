"""CPU-side checks of the C-ABI library: it loads, exports every entry point
the header declares, its struct layout matches the binding, and invalid
arguments are rejected before any HIP call (so these run without a GPU)."""
import ctypes
import os
import re
import subprocess

import pytest

import combine_get_dispatch_scan_amd as ep

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "moe_ep.h")


def _declared():
    src = open(HEADER).read()
    src = re.sub(r"/\*.*?\*/", "", src, flags=re.S)
    return sorted(set(re.findall(r"\b(ep_[a-z0-9_]+)\s*\(", src)))


def test_library_exports_every_declared_symbol():
    lib = ep.load()
    names = _declared()
    assert len(names) >= 9
    for n in names:
        assert hasattr(lib, n), n
        assert n in ep._SIGS, f"binding lacks {n}"
        assert callable(getattr(ep, n)), n


def test_handle_layout_matches_c(tmp_path):
    fields = [f for f, _ in ep.ep_handle_t._fields_]
    prog = "#include <stdio.h>\n#include <stddef.h>\n#include \"moe_ep.h\"\nint main(void){\n"
    prog += 'printf("%zu\\n", sizeof(ep_handle_t));\n'
    for f in fields:
        prog += f'printf("%zu\\n", offsetof(ep_handle_t, {f}));\n'
    prog += "return 0;}\n"
    c = tmp_path / "layout.c"
    c.write_text(prog)
    exe = tmp_path / "layout"
    subprocess.run(["gcc", "-D__HIP_PLATFORM_AMD__", "-I", os.path.join(ROOT, "include"),
                    "-I", "/opt/rocm/include", str(c), "-o", str(exe)], check=True)
    vals = [int(v) for v in subprocess.run([str(exe)], capture_output=True, text=True,
                                           check=True).stdout.split()]
    assert vals[0] == ctypes.sizeof(ep.ep_handle_t)
    for f, off in zip(fields, vals[1:]):
        assert getattr(ep.ep_handle_t, f).offset == off, f


def test_version_and_workspace_size():
    assert ep.ep_version() >= 10000
    assert ep.ep_workspace_bytes(0, 8, 256, 8) > 0
    a = ep.ep_workspace_bytes(8192, 8, 256, 8)
    b = ep.ep_workspace_bytes(16384, 8, 256, 16)
    assert b > a > 0
    # at least slot + src_token + weights + pair codes
    assert a >= 4 * 8192 * 8 * 4
    for bad in [(-1, 8, 256, 8), (10, 0, 256, 8), (10, 17, 256, 8), (10, 8, 0, 1),
                (10, 8, 1025, 1), (10, 8, 256, 7), (10, 8, 256, 128), (1 << 28, 16, 64, 8)]:
        assert ep.ep_workspace_bytes(*bad) == 0, bad


FAKE = 1 << 20  # never dereferenced: every call below fails validation first


def _layout_args(**kw):
    a = dict(topk_idx=FAKE, num_tokens=64, num_topk=4, num_experts=16, num_partitions=4,
             num_tokens_per_partition=FAKE, num_tokens_per_expert=FAKE,
             is_token_in_partition=FAKE, num_invalid=FAKE, ws=FAKE,
             ws_bytes=ep.ep_workspace_bytes(64, 4, 16, 4), handle=ep.ep_handle_t(), stream=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,msg", [
    (dict(num_partitions=3), "invalid dims"),
    (dict(num_topk=17), "invalid dims"),
    (dict(num_experts=2048, num_partitions=8), "invalid dims"),
    (dict(num_tokens=-5), "invalid dims"),
    (dict(topk_idx=None), "topk_idx"),
    (dict(topk_idx=FAKE + 4), "topk_idx"),
    (dict(is_token_in_partition=None), "is_token_in_partition"),
    (dict(num_invalid=None), "count outputs"),
    (dict(num_tokens_per_expert=FAKE + 2), "count outputs"),
    (dict(ws=None), "workspace"),
    (dict(ws=FAKE + 64), "workspace"),
    (dict(ws_bytes=100), "workspace too small"),
])
def test_layout_rejects_invalid_arguments(kw, msg):
    a = _layout_args(**kw)
    rc = ep.ep_get_dispatch_layout(**a)
    assert rc == ep.EP_EINVAL
    assert msg in ep.ep_last_error()
    assert a["handle"].magic == 0


def test_layout_rejects_null_handle():
    a = _layout_args()
    lib = ep.load()
    rc = lib.ep_get_dispatch_layout(a["topk_idx"], 64, 4, 16, 4, FAKE, FAKE, FAKE, FAKE, FAKE,
                                    a["ws_bytes"], None, None)
    assert rc == ep.EP_EINVAL and "handle" in ep.ep_last_error()


def _fake_handle(stage=1, T=64, K=4, E=16, P=4):
    h = ep.ep_handle_t()
    h.magic = ep.EP_HANDLE_MAGIC
    h.stage = stage
    h.num_tokens, h.num_topk, h.num_experts, h.num_partitions = T, K, E, P
    h.hidden, h.use_fp8, h.capacity_rows = 256, 1, T * K
    return h


@pytest.mark.parametrize("kw,msg", [
    (dict(hidden=0), "hidden"),
    (dict(hidden=100), "hidden"),
    (dict(hidden=65536), "hidden"),
    (dict(hidden=136, use_fp8=1), "hidden % 128"),
    (dict(use_fp8=2), "use_fp8"),
    (dict(capacity_rows=-1), "capacity_rows"),
    (dict(capacity_rows=64 * 4 + 1), "capacity_rows"),
    (dict(x=None), "x must"),
    (dict(x=FAKE + 8), "x must"),
    (dict(recv_x=FAKE + 4), "recv_x"),
    (dict(recv_scales=None), "recv_scales"),
    (dict(topk_weights=FAKE + 2), "topk_weights"),
])
def test_dispatch_rejects_invalid_arguments(kw, msg):
    a = dict(x=FAKE, topk_weights=FAKE, hidden=256, use_fp8=1, recv_x=FAKE, recv_scales=FAKE,
             capacity_rows=64 * 4, handle=_fake_handle(), stream=None)
    a.update(kw)
    rc = ep.ep_dispatch(**a)
    assert rc == ep.EP_EINVAL, ep.ep_last_error()
    assert msg in ep.ep_last_error()
    assert a["handle"].stage == 1


def test_calls_need_the_right_stage():
    h = ep.ep_handle_t()
    assert ep.ep_dispatch(FAKE, FAKE, 256, 0, FAKE, None, 10, h, None) == ep.EP_EINVAL
    assert "ep_get_dispatch_layout" in ep.ep_last_error()
    h1 = _fake_handle(stage=1)
    assert ep.ep_dispatch_cached(FAKE, h1, FAKE, FAKE, None) == ep.EP_EINVAL
    assert "dispatched" in ep.ep_last_error()
    assert ep.ep_combine(FAKE, h1, FAKE, FAKE, None) == ep.EP_EINVAL
    h2 = _fake_handle(stage=2)
    h2.has_weights = 0
    assert ep.ep_combine(FAKE, h2, None, FAKE, None) == ep.EP_EINVAL
    assert "no weights" in ep.ep_last_error()
    assert ep.ep_combine(FAKE + 8, h2, FAKE, FAKE, None) == ep.EP_EINVAL
    assert ep.ep_combine(FAKE, h2, FAKE, FAKE + 8, None) == ep.EP_EINVAL
    assert ep.ep_handle_recv_counts(ep.ep_handle_t(), None, None, None) == ep.EP_EINVAL
    assert ep.ep_e4m3fn_encode(None, None, -1, None) == ep.EP_EINVAL
    assert ep.ep_e4m3fn_encode(None, FAKE, 10, None) == ep.EP_EINVAL


def test_product_path_never_imports_the_oracle():
    pkg = os.path.join(ROOT, "combine_get_dispatch_scan_amd")
    for dirpath, _, files in os.walk(pkg):
        for f in files:
            if f.endswith((".py", ".hip", ".h", ".cpp")):
                src = open(os.path.join(dirpath, f)).read()
                assert "oracle" not in src.lower(), f


def test_recv_counts_decode_on_host():
    """ep_recv_counts_decode is host-only: counts are offset differences, the
    status words select the return code."""
    E = 6
    h = _fake_handle(stage=2, E=E, P=3)
    h.capacity_rows = 9
    h.dispatch_seq = 1
    off = [0, 3, 4, 5, 7, 7, 9]
    for status, want in [([0, 0, 9, 0], ep.EP_OK), ([1, 0, 9, 0], ep.EP_ECAPACITY),
                         ([0, 2, 9, 0], ep.EP_EIDS), ([1, 2, 9, 0], ep.EP_ECAPACITY)]:
        buf = (ctypes.c_int32 * (E + 5))(*(off + status))
        counts = (ctypes.c_int32 * E)()
        n = ctypes.c_int32(-1)
        rc = ep.ep_recv_counts_decode(h, buf, counts, ctypes.byref(n))
        assert rc == want, (status, rc)
        assert list(counts) == [3, 1, 1, 2, 0, 2] and n.value == 9
    # a dense layout's drops also follow from N > capacity_rows (a copy taken
    # before dispatch set the flag); aligned layouts rely on the flag alone
    h.capacity_rows = 8
    buf = (ctypes.c_int32 * (E + 5))(*(off + [0, 0, 9, 0]))
    assert ep.ep_recv_counts_decode(h, buf, None, None) == ep.EP_ECAPACITY
    h.expert_alignment = 4
    assert ep.ep_recv_counts_decode(h, buf, None, None) == ep.EP_OK
    h.expert_alignment = 1
    h.static_cap = 3
    assert ep.ep_recv_counts_decode(h, buf, None, None) == ep.EP_OK
    # the overflow word counts only when it holds the handle's latest
    # dispatch number: a mark left by dispatch 1 is stale once dispatch 2 ran
    h.static_cap = 0
    h.capacity_rows = 9
    h.dispatch_seq = 2
    for mark, want in [(1, ep.EP_OK), (2, ep.EP_ECAPACITY), (3, ep.EP_OK)]:
        buf = (ctypes.c_int32 * (E + 5))(*(off + [mark, 0, 9, 0]))
        assert ep.ep_recv_counts_decode(h, buf, None, None) == want, mark
    h.expert_alignment = 4
    buf = (ctypes.c_int32 * (E + 5))(*(off + [1, 0, 9, 0]))
    assert ep.ep_recv_counts_decode(h, buf, None, None) == ep.EP_OK
    h.expert_alignment = 1
    # before dispatch the overflow word is not consulted
    h1 = _fake_handle(stage=1, E=E, P=3)
    buf = (ctypes.c_int32 * (E + 5))(*(off + [1, 0, 9, 0]))
    assert ep.ep_recv_counts_decode(h1, buf, None, None) == ep.EP_OK
    assert ep.ep_recv_counts_decode(h1, None, None, None) == ep.EP_EINVAL
    assert ep.ep_handle_recv_counts_async(h1, None, None) == ep.EP_EINVAL
    assert ep.ep_handle_recv_counts_async(ep.ep_handle_t(), FAKE, None) == ep.EP_EINVAL


def test_backward_calls_validate_before_any_hip_call():
    h1 = _fake_handle(stage=1)
    assert ep.ep_dispatch_backward(FAKE, h1, FAKE, None) == ep.EP_EINVAL
    assert ep.ep_combine_backward(FAKE, FAKE, h1, FAKE, FAKE, FAKE, None) == ep.EP_EINVAL
    h2 = _fake_handle(stage=2)
    h2.hidden = 256
    assert ep.ep_dispatch_backward(FAKE, h2, FAKE + 8, None) == ep.EP_EINVAL
    assert "grad_x" in ep.ep_last_error()
    assert ep.ep_dispatch_backward(FAKE + 4, h2, FAKE, None) == ep.EP_EINVAL
    assert "grad_recv" in ep.ep_last_error()
    h2.has_weights = 0
    assert ep.ep_combine_backward(FAKE, FAKE, h2, None, FAKE, FAKE, None) == ep.EP_EINVAL
    assert "no weights" in ep.ep_last_error()
    assert ep.ep_combine_backward(FAKE + 8, FAKE, h2, FAKE, FAKE, FAKE, None) == ep.EP_EINVAL
    assert "grad_out" in ep.ep_last_error()
    assert ep.ep_combine_backward(FAKE, FAKE, h2, FAKE, None, FAKE, None) == ep.EP_EINVAL
    assert "grad_y" in ep.ep_last_error()
    assert ep.ep_combine_backward(FAKE, None, h2, FAKE, FAKE, FAKE, None) == ep.EP_EINVAL
    assert "needs y" in ep.ep_last_error()
    assert ep.ep_combine_backward(FAKE, FAKE, h2, FAKE, FAKE, FAKE + 2, None) == ep.EP_EINVAL


def _ll_args(**kw):
    T, K, E, P = 32, 4, 16, 4
    a = dict(x=FAKE, topk_idx=FAKE, topk_weights=FAKE, num_tokens=T, hidden=256, num_topk=K,
             num_experts=E, num_partitions=P, use_fp8=1, num_max_tokens=8, recv_x=FAKE,
             recv_scales=FAKE, num_tokens_per_partition=FAKE, num_tokens_per_expert=FAKE,
             is_token_in_partition=FAKE, num_invalid=FAKE, ws=FAKE,
             ws_bytes=ep.ep_workspace_bytes(T, K, E, P), handle=ep.ep_handle_t(), stream=None)
    a.update(kw)
    return a


@pytest.mark.parametrize("kw,msg", [
    (dict(num_tokens=257), "at most 256"),
    (dict(num_tokens=-1), "invalid dims"),
    (dict(num_max_tokens=0), "num_max_tokens"),
    (dict(num_max_tokens=1 << 30), "num_max_tokens"),
    (dict(num_experts=15), "invalid dims"),
    (dict(topk_idx=None), "topk_idx"),
    (dict(topk_idx=FAKE + 4), "topk_idx"),
    (dict(is_token_in_partition=None), "is_token_in_partition"),
    (dict(num_invalid=None), "count outputs"),
    (dict(topk_weights=FAKE + 2), "topk_weights"),
    (dict(ws=FAKE + 16), "workspace"),
    (dict(ws_bytes=64), "workspace too small"),
    (dict(hidden=100), "hidden"),
    (dict(hidden=136), "hidden % 128"),
    (dict(use_fp8=2), "use_fp8"),
    (dict(x=None), "x must"),
    (dict(recv_x=FAKE + 8), "recv_x"),
    (dict(recv_scales=None), "recv_scales"),
    (dict(handle=None), "handle"),
])
def test_low_latency_dispatch_rejects_invalid_arguments(kw, msg):
    a = _ll_args(**kw)
    h = a["handle"]
    if a["handle"] is None:
        rc = ep.load().ep_low_latency_dispatch(*[a[k] for k in list(a)[:-2]], None, None)
    else:
        rc = ep.ep_low_latency_dispatch(**a)
    assert rc == ep.EP_EINVAL, ep.ep_last_error()
    assert msg in ep.ep_last_error(), ep.ep_last_error()
    if h is not None:
        assert h.magic == 0, "handle written on an error path"


def test_static_handle_is_refused_by_fresh_dispatch():
    h = _fake_handle(stage=2)
    h.static_cap = 8
    rc = ep.ep_dispatch(FAKE, FAKE, 256, 1, FAKE, FAKE, 16 * 8, h, None)
    assert rc == ep.EP_EINVAL and "ep_dispatch_cached" in ep.ep_last_error()
    # the cached call accepts E*cap rows for a static handle, and no more
    h.capacity_rows = 16 * 8 + 1
    assert ep.ep_dispatch_cached(FAKE, h, FAKE, FAKE, None) == ep.EP_EINVAL
    assert "capacity_rows" in ep.ep_last_error()


def test_fp8_combine_calls_validate_before_any_hip_call():
    h1 = _fake_handle(stage=1)
    assert ep.ep_combine_fp8(FAKE, FAKE, h1, FAKE, FAKE, None) == ep.EP_EINVAL
    assert ep.ep_dispatch_backward_fp8(FAKE, FAKE, h1, FAKE, None) == ep.EP_EINVAL
    h2 = _fake_handle(stage=2)
    for args, msg in [((FAKE + 8, FAKE, h2, FAKE, FAKE), "FP8 rows"),
                      ((FAKE, None, h2, FAKE, FAKE), "FP8 scales"),
                      ((FAKE, FAKE + 2, h2, FAKE, FAKE), "FP8 scales"),
                      ((FAKE, FAKE, h2, FAKE, FAKE + 8), "out"),
                      ((FAKE, FAKE, h2, FAKE + 2, FAKE), "topk_weights")]:
        assert ep.ep_combine_fp8(*args, None) == ep.EP_EINVAL
        assert msg in ep.ep_last_error(), (msg, ep.ep_last_error())
    h2.has_weights = 0
    assert ep.ep_combine_fp8(FAKE, FAKE, h2, None, FAKE, None) == ep.EP_EINVAL
    assert "no weights" in ep.ep_last_error()
    assert ep.ep_dispatch_backward_fp8(FAKE, FAKE, h2, FAKE + 8, None) == ep.EP_EINVAL
    assert "grad_x" in ep.ep_last_error()
    h2.hidden = 136
    assert ep.ep_dispatch_backward_fp8(FAKE, FAKE, h2, FAKE, None) == ep.EP_EINVAL
    assert "hidden % 128" in ep.ep_last_error()


def test_noalloc_scratch_covers_every_low_latency_call():
    """The allocation-free dispatch's per-GPU array holds the handle arrays
    of the largest low-latency call the limits allow, the header and the
    binding agree on its size, and arguments are checked before any HIP call."""
    hdr = open(os.path.join(ROOT, "include", "moe_ep.h")).read()
    assert re.search(r"#define EP_NOALLOC_SCRATCH_BYTES\s+(\d+)", hdr).group(1) == str(ep.EP_NOALLOC_SCRATCH_BYTES)
    assert re.search(r"#define EP_MAX_LL_TOKENS\s+(\d+)", hdr).group(1) == str(ep.EP_MAX_LL_TOKENS)
    need = ep.ep_workspace_bytes(ep.EP_MAX_LL_TOKENS, 16, 1024, 64)
    assert 0 < need <= ep.EP_NOALLOC_SCRATCH_BYTES, need
    h = ep.ep_handle_t()
    for args in [(300, 128, 2, 8, 2, 0, 4), (16, 128, 2, 8, 3, 0, 4), (16, 100, 2, 8, 2, 1, 4),
                 (16, 128, 2, 8, 2, 0, 0)]:
        T, H, K, E, P, fp8, cap = args
        rc = ep.ep_low_latency_dispatch_noalloc(FAKE, FAKE, None, T, H, K, E, P, fp8, cap, FAKE, FAKE,
                                                FAKE, FAKE, FAKE, FAKE, h, None)
        assert rc == ep.EP_EINVAL, args
        assert ep.ep_last_error()
