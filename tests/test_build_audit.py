"""Build audit (CPU): the compiler's resource-usage remarks for every kernel
of the library, built for gfx950 with the library's own flags.  No kernel
spills VGPRs or uses scratch; the score kernel runs one wave per SIMD with
q in the 256 AGPRs."""
import os
import re
import shutil
import subprocess

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "fp8_key_scoring_amd", "csrc")
HIPCC = "/opt/rocm/bin/hipcc"


def _remarks(src):
    cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-Xclang", "-target-feature", "-Xclang",
           "-packed-fp32-ops", "-mllvm", "-amdgpu-mfma-vgpr-form", "-Rpass-analysis=kernel-resource-usage",
           "-I", os.path.join(ROOT, "include"), "-I", CSRC, "--cuda-device-only", "-c", src, "-o", os.devnull]
    out = subprocess.run(cmd, capture_output=True, text=True, timeout=600)
    assert out.returncode == 0, out.stderr[-2000:]
    kernels, cur = {}, None
    for line in out.stderr.splitlines():
        m = re.search(r"remark:\s+(.*?)\s*\[-Rpass-analysis", line)
        if not m:
            continue
        text = m.group(1)
        if text.startswith("Function Name:"):
            cur = text.split(":", 1)[1].strip()
            kernels[cur] = {}
        elif cur and ":" in text:
            k, v = text.split(":", 1)
            kernels[cur][k.strip()] = v.strip()
    return kernels


@pytest.mark.skipif(not os.path.exists(HIPCC) and shutil.which("hipcc") is None, reason="hipcc not installed")
def test_no_spills_or_scratch_and_score_kernel_occupancy():
    seen = {}
    for f in sorted(os.listdir(CSRC)):
        if f.endswith(".hip") and f != "api.hip":
            seen.update(_remarks(os.path.join(CSRC, f)))
    assert any("score_kernel" in k for k in seen) and any("finalize_kernel" in k for k in seen)
    for name, r in seen.items():
        assert r["VGPRs Spill"] == "0", (name, r)
        assert r["ScratchSize [bytes/lane]"] == "0", (name, r)
    for name, r in seen.items():
        if "score_kernel" in name:
            assert r["AGPRs"] == "256" and r["Occupancy [waves/SIMD]"] == "1", (name, r)
