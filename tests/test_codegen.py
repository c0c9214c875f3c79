"""Generated-code checks (CPU: hipcc cross-compiles for gfx950, nothing runs).

The combine kernels are bandwidth-bound only while each wave keeps its K row
gathers in flight together.  With the weight fixed at 1.0, the predicated
form of the FP8 combine once compiled to a full wait (`s_waitcnt vmcnt(0)`)
ahead of every row load, one gather at a time per wave, and ran 20% slower.
These tests compile the combine source with the library's own flags and
check, in the assembly, that no 16-byte row load of the hot-path
instantiations sits right behind such a wait.
"""
import os
import re
import shutil
import subprocess

import pytest

from combine_get_dispatch_scan_amd import _build

# instantiations with K <= 8 on the forward and backward paths
KERNELS = {
    "combine_kernel<8, weighted, sc1 stores>": "_ZN6moe_ep14combine_kernelILi8ELb0ELi16EEEvNS_11CombineArgsE",
    "combine_kernel<8, unit, sc1 stores>": "_ZN6moe_ep14combine_kernelILi8ELb1ELi16EEEvNS_11CombineArgsE",
    "combine_kernel<8, weighted, nt stores>": "_ZN6moe_ep14combine_kernelILi8ELb0ELi2EEEvNS_11CombineArgsE",
    "combine_fp8_kernel<8, weighted>": "_ZN6moe_ep18combine_fp8_kernelILi8ELb0ELb0EEEvNS_14CombineFp8ArgsE",
    "combine_fp8_kernel<8, unit, row buffers>": "_ZN6moe_ep18combine_fp8_kernelILi8ELb1ELb1EEEvNS_14CombineFp8ArgsE",
    "combine_fp8_kernel<4, unit, row buffers>": "_ZN6moe_ep18combine_fp8_kernelILi4ELb1ELb1EEEvNS_14CombineFp8ArgsE",
    "combine_owner_kernel<8, weighted, nt|sc1 stores>": "_ZN6moe_ep20combine_owner_kernelILi8ELb0ELi18EEEvNS_11CombineArgsE",
    "combine_owner_kernel<8, unit, nt|sc1 stores>": "_ZN6moe_ep20combine_owner_kernelILi8ELb1ELi18EEEvNS_11CombineArgsE",
}

ROW_LOAD = re.compile(r"^(global_load_dwordx4|buffer_load_dwordx4)\b")


@pytest.fixture(scope="module")
def combine_asm(tmp_path_factory):
    if not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    out = tmp_path_factory.mktemp("asm") / "combine.s"
    flags = [f for f in _build.FLAGS if f not in ("-shared", "-fPIC")]
    cmd = [_build.HIPCC, *flags, "--cuda-device-only", "-S", "-I", _build.INCLUDE, "-I", _build.CSRC,
           os.path.join(_build.CSRC, "combine.hip"), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _body(asm, symbol):
    assert symbol + ":" in asm, (f"{symbol} is not in the compiled combine.hip: the kernel's "
                                 "template or argument list changed; update KERNELS")
    start = asm.index(symbol + ":")
    end = asm.index("s_endpgm", start)
    lines = [l.strip() for l in asm[start:end].splitlines()]
    return [l for l in lines if l and not l.startswith((";", "."))]


@pytest.mark.parametrize("name", sorted(KERNELS))
def test_row_gathers_are_not_serialised(combine_asm, name):
    body = _body(combine_asm, KERNELS[name])
    loads = [i for i, l in enumerate(body) if ROW_LOAD.match(l)]
    assert len(loads) >= 4, f"{name}: expected the K row gathers in the body"
    waited = [i for i in loads
              if any(l.startswith("s_waitcnt vmcnt(0)") for l in body[max(0, i - 3):i])]
    assert not waited, (f"{name}: {len(waited)} of {len(loads)} row gathers wait for all "
                        f"earlier loads first:\n" + "\n".join(body[i] for i in waited[:4]))


# ----------------------------------------------------------------------------
# no packed fp32 arithmetic in the device code
# ----------------------------------------------------------------------------

PACKED_F32 = re.compile(r"\bv_pk_[a-z0-9_]*_f32\b")

# float2 arithmetic that hipcc -O3 turns into packed fp32 instructions for
# gfx950 unless the target feature is switched off
PK_PROBE = r"""
#include <hip/hip_runtime.h>
__global__ void probe(const float2* __restrict__ a, const float2* __restrict__ b,
                      float2* __restrict__ o, int n)
{
    int i = blockIdx.x * blockDim.x + threadIdx.x;
    if (i < n) {
        float2 x = a[i], y = b[i], r;
        r.x = (x.x * y.x + 1.5f) * x.x;
        r.y = (x.y * y.y + 1.5f) * x.y;
        o[i] = r;
    }
}
"""


def _device_asm(src, out, flags):
    cmd = [_build.HIPCC, *flags, "--cuda-device-only", "-S", "-I", _build.INCLUDE, "-I", _build.CSRC,
           str(src), "-o", str(out)]
    subprocess.run(cmd, check=True, capture_output=True)
    return out.read_text()


def _asm_flags():
    return [f for f in _build.FLAGS if f not in ("-shared", "-fPIC")]


def test_packed_fp32_flag_takes_effect_on_the_device(tmp_path):
    """The host pass of hipcc warns that it does not know the packed-fp32
    feature; the device pass honours it: the probe compiles to packed fp32
    instructions without the flag and to none with the library's flags."""
    if not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    src = tmp_path / "probe.hip"
    src.write_text(PK_PROBE)
    flags = _asm_flags()
    i = flags.index("-packed-fp32-ops")
    without = flags[:i - 3] + flags[i + 1:]           # drop "-Xclang -target-feature -Xclang -packed-fp32-ops"
    assert "-packed-fp32-ops" not in without and len(without) == len(flags) - 4
    assert PACKED_F32.search(_device_asm(src, tmp_path / "a.s", without)), \
        "the probe no longer makes packed fp32 code without the flag: pick another probe"
    assert not PACKED_F32.search(_device_asm(src, tmp_path / "b.s", flags))


def test_no_packed_fp32_in_any_kernel(tmp_path):
    """Every HIP source, compiled for gfx950 with the library's flags, holds no
    packed fp32 instruction (v_pk_add_f32, v_pk_mul_f32, v_pk_fma_f32, ...)."""
    if not os.path.exists(_build.HIPCC) and shutil.which("hipcc") is None:
        pytest.skip("hipcc not available")
    kernels = 0
    for src in _build.sources():
        asm = _device_asm(src, tmp_path / (os.path.basename(src) + ".s"), _asm_flags())
        kernels += asm.count(".amdhsa_kernel ")
        hits = sorted(set(PACKED_F32.findall(asm)))
        assert not hits, f"{os.path.basename(src)}: {hits}"
    assert kernels >= 40, kernels         # every kernel instantiation was looked at
