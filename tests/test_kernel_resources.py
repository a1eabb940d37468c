"""Compile-time resource checks of the HIP kernels (CPU only; hipcc
cross-compiles for gfx950): no kernel may use scratch memory (a spilled
register or an argument struct copied to the stack costs far more than any
change that caused it) and none may exceed the 512 registers of a SIMD lane.
These regressions are silent at run time apart from speed."""

import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "long_context_sparse_static_amd", "csrc")
HIPCC = os.environ.get("HIPCC") or shutil.which("hipcc") or "/opt/rocm/bin/hipcc"
SOURCES = ["fwd_bf16.hip", "bwd_bf16.hip", "decode_bf16.hip", "fwd_f32.hip"]


def kernel_resources(src, tmp_path):
    cmd = [HIPCC, "-x", "hip", "-O3", "-std=c++17", "--offload-arch=gfx950", "--cuda-device-only",
           "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops",
           "-I", os.path.join(ROOT, "include"), "-c", os.path.join(CSRC, src),
           "-o", str(tmp_path / (src + ".o")), "-Rpass-analysis=kernel-resource-usage"]
    r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, r.stderr[-2000:]
    out, cur = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            cur = m.group(1)
            out[cur] = {}
            continue
        m = re.search(r"remark:\s+(VGPRs|AGPRs|ScratchSize \[bytes/lane\]): (\d+)", line)
        if m and cur:
            out[cur][m.group(1).split()[0]] = int(m.group(2))
    return out


@pytest.mark.skipif(not os.path.exists(HIPCC), reason="hipcc not available")
@pytest.mark.parametrize("src", SOURCES)
def test_no_scratch_and_registers_fit(src, tmp_path):
    res = kernel_resources(src, tmp_path)
    kernels = {k: v for k, v in res.items() if "kernel" in k}
    assert kernels, "no kernels reported"
    for name, r in kernels.items():
        # every figure must have been read: a report format the parser does
        # not match would otherwise pass vacuously
        assert {"VGPRs", "AGPRs", "ScratchSize"} <= set(r), f"{name}: resource report not parsed: {r}"
        assert r["ScratchSize"] == 0, f"{name} uses {r['ScratchSize']} bytes of scratch per lane"
        assert r.get("VGPRs", 0) + r.get("AGPRs", 0) <= 512, f"{name} uses too many registers: {r}"
