"""The FP8 attention kernel's loop shapes other than the default (one stage, four waves) are
selected at build time (ATTN_FP8_SHAPE) for ablation runs.  This CPU test cross-compiles fp8.hip
for gfx950 with each of them and checks that they still build and that no instance spills
registers to scratch memory (a spilling loop shape would measure the spills, not the schedule)."""
from __future__ import annotations

import concurrent.futures
import os
import re
import shutil
import subprocess
import tempfile

import pytest

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_76_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

SHAPES = {
    "one stage, 4 waves (default)": "4,64,kLoopOne",
    "two-stage, 4 waves": "4,64,kLoopTwoStage",
    "two-stage, 8 waves": "8,64,kLoopTwoStage",
    "ping-pong, 8 waves": "8,64,kLoopPingPong",
}


def _scratch_per_kernel(shape: str) -> dict[str, int]:
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", f"-DATTN_FP8_SHAPE={shape}",
               "--cuda-device-only", "-c", os.path.join(CSRC, "fp8.hip"), "-o", os.path.join(tmp, "fp8.o"),
               "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed for ATTN_FP8_SHAPE={shape}:\n{r.stderr[-3000:]}"
    scratch, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
        m = re.search(r"ScratchSize \[bytes/lane\]: (\d+)", line)
        if m and name:
            scratch[name] = int(m.group(1))
    return scratch


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_fp8_loop_shapes_build_without_spills():
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SHAPES)) as ex:
        results = dict(zip(SHAPES, ex.map(_scratch_per_kernel, SHAPES.values())))
    for label, scratch in results.items():
        attn = {k: v for k, v in scratch.items() if "fwd_fp8_kernel" in k}
        assert len(attn) == 6, f"{label}: expected 6 attention kernel instances, found {len(attn)}"
        spilled = {k: v for k, v in attn.items() if v}
        assert not spilled, f"{label}: instances with scratch memory (register spills): {spilled}"
