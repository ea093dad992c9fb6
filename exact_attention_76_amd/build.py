"""Build libattn.so (the attention path: api, attn_fwd, fp8) and libceiling.so (the matrix-core
throughput probe that bench.py reports beside the attention figures) for gfx950 with hipcc."""
from __future__ import annotations

import concurrent.futures
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
SOURCES = ["api.hip", "attn_fwd.hip", "attn_bwd.hip", "fp8.hip"]
CEILING_LIB = os.path.join(PKG, "libceiling.so")
CEILING_SOURCES = ["ceiling.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: hipcc must not form v_pk_{add,mul,fma}_f32 from scalar or float2 code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
# Extra compiler arguments (whitespace-separated), e.g. a different loop shape for an ablation run:
#   ATTN_HIPCC_EXTRA='-DATTN_D128_SHAPE=64,attn::LoopShape<8,true>' python exact_attention_76_amd/build.py
FLAGS += os.environ.get("ATTN_HIPCC_EXTRA", "").split()


def _compile(src: str) -> str:
    obj = os.path.join(OBJ_DIR, os.path.splitext(src)[0] + ".o")
    cmd = [HIPCC, *FLAGS, "-c", os.path.join(CSRC, src), "-o", obj]
    r = subprocess.run(cmd, capture_output=True, text=True)
    errs = "\n".join(l for l in r.stderr.splitlines() if "packed-fp32-ops" not in l)
    if r.returncode != 0:
        raise RuntimeError(f"hipcc failed on {src}:\n{errs}")
    if errs.strip():
        sys.stderr.write(errs + "\n")
    return obj


def _link(objs: list[str], lib: str) -> None:
    tmp = lib + ".tmp"
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-shared", "-fPIC", "-o", tmp, *objs], check=True)
    os.replace(tmp, lib)


def build() -> str:
    """Compile every source (in parallel) and link libattn.so and libceiling.so in the package
    directory; returns the path of libattn.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    sources = SOURCES + CEILING_SOURCES
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(sources)) as ex:
        objs = dict(zip(sources, ex.map(_compile, sources)))
    _link([objs[s] for s in SOURCES], LIB)
    _link([objs[s] for s in CEILING_SOURCES], CEILING_LIB)
    return LIB


if __name__ == "__main__":
    print(build())
