"""Build-level properties of the HIP library, checked on the CPU (hipcc cross-compiles gfx950)."""
import os
import re
import subprocess

import pytest

from sparse_attention_10_amd import build

CSRC = os.path.join(os.path.dirname(build.__file__), "csrc")


@pytest.mark.parametrize("debug", [False, True], ids=["release", "debug"])
@pytest.mark.parametrize("src", build.SOURCES)
def test_no_kernel_needs_scratch(src, debug, tmp_path):
    """Every kernel fits its registers: no private (scratch) segment, no dynamic stack; the same
    for the DSA_DEBUG build, whose checks add only compares and atomic flag writes."""
    if src == "api.hip":
        pytest.skip("host-side validation only")
    out = tmp_path / "k.s"
    cmd = ([build.hipcc()] + build.flags() + (["-DDSA_DEBUG"] if debug else []) +
           ["--cuda-device-only", "-S", os.path.join(CSRC, src), "-o", str(out)])
    subprocess.run(cmd, check=True, capture_output=True)
    text = out.read_text()
    kernels = re.findall(r"\.amdhsa_kernel (\S+)", text)
    assert kernels
    sizes = [int(x) for x in re.findall(r"\.amdhsa_private_segment_fixed_size (\d+)", text)]
    dyn = [int(x) for x in re.findall(r"\.amdhsa_uses_dynamic_stack (\d+)", text)]
    assert len(sizes) == len(kernels) and all(v == 0 for v in sizes), dict(zip(kernels, sizes))
    assert all(v == 0 for v in dyn)
    # built without packed-fp32 VALU forms
    assert "-packed-fp32-ops" in build.flags()
    assert not re.search(r"v_pk_(add|mul|fma)_f32", text)
