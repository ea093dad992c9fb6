"""Every kernel instance of the library cross-compiles for gfx950 without spilling registers to
scratch memory (a CPU test: hipcc's device pass only).  A spill would put per-lane stack traffic
on the hot path, so each default loop shape is sized to fit its register budget; this test keeps
it that way."""
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

# source file -> (kernel name fragment, number of instances the dispatch builds)
KERNELS = {
    # bf16/fp16 x (d 64/128/256 x (4 modes + 2 windowed) + the short non-causal d = 128 shape x 2 modes
    # + the persistent non-causal dense d = 128 shape)
    "attn_fwd.hip": ("fwd_kernel", 2 * (3 * 6 + 2 + 1)),
    "fp8.hip": ("fwd_fp8_kernel", 6),            # 4 modes + 2 windowed
    "attn_bwd.hip": ("bwd_", None),
}
# Known, bounded exceptions (bytes of scratch per lane): the causal d = 128 dK/dV kernels, whose
# tile loop is unrolled by two, park one register across the loop -- one store before it, one
# load in the epilogue, none inside the loop.
ALLOWED_SCRATCH = {r"bwd_dkdv_kernelILi128ELb[01]ELb1E": 8}


def _resources(src: str) -> dict[str, dict[str, int]]:
    with tempfile.TemporaryDirectory() as tmp:
        cmd = [HIPCC, "--offload-arch=gfx950", "-O3", "-std=c++17", "-I", os.path.join(ROOT, "include"), "-I", CSRC,
               "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "--cuda-device-only", "-c",
               os.path.join(CSRC, src), "-o", os.path.join(tmp, "k.o"), "-Rpass-analysis=kernel-resource-usage"]
        r = subprocess.run(cmd, capture_output=True, text=True)
    assert r.returncode == 0, f"hipcc failed for {src}:\n{r.stderr[-3000:]}"
    out, name = {}, None
    for line in r.stderr.splitlines():
        m = re.search(r"Function Name: (\S+)", line)
        if m:
            name = m.group(1)
            out[name] = {}
        m = re.search(r"(ScratchSize \[bytes/lane\]|VGPRs|AGPRs): (\d+)", line)
        if m and name:
            out[name][m.group(1)] = int(m.group(2))
    return out


@pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC), reason="hipcc not available")
def test_kernels_build_without_spills():
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(KERNELS)) as ex:
        results = dict(zip(KERNELS, ex.map(_resources, KERNELS)))
    for src, (frag, count) in KERNELS.items():
        kern = {k: v for k, v in results[src].items() if frag in k}
        if count is not None:
            assert len(kern) == count, f"{src}: expected {count} {frag} instances, found {len(kern)}"
        assert kern, f"{src}: no {frag} instances"
        spilled = {k: v["ScratchSize [bytes/lane]"] for k, v in kern.items() if v.get("ScratchSize [bytes/lane]")
                   and not any(re.search(p, k) and v["ScratchSize [bytes/lane]"] <= b
                               for p, b in ALLOWED_SCRATCH.items())}
        assert not spilled, f"{src}: instances with scratch memory (register spills): {spilled}"
