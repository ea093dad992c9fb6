"""Build libattn.so (the attention path: api, attn_fwd, attn_bwd, fp8) for gfx950 with hipcc.

Beside the library, build() writes libattn.so.sources.json: the sha256 of every source file the
library was compiled from (csrc/*, include/attn.h) and the extra compiler arguments.
load_library() refuses a library whose record does not match the sources on disk, so the tests,
the smoke check and the benchmark always run the code that is in the tree."""
from __future__ import annotations

import concurrent.futures
import hashlib
import json
import os
import subprocess
import sys

PKG = os.path.dirname(os.path.abspath(__file__))
ROOT = os.path.dirname(PKG)
CSRC = os.path.join(PKG, "csrc")
INCLUDE = os.path.join(ROOT, "include")
OBJ_DIR = os.path.join(PKG, "_build")
LIB = os.path.join(PKG, "libattn.so")
RECORD = LIB + ".sources.json"
SOURCES = ["api.hip", "attn_fwd.hip", "attn_bwd.hip", "fp8.hip"]
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")

# -packed-fp32-ops: hipcc must not form v_pk_{add,mul,fma}_f32 from scalar or float2 code.
FLAGS = ["--offload-arch=gfx950", "-O3", "-std=c++17", "-fPIC", "-I", INCLUDE, "-I", CSRC,
         "-Xclang", "-target-feature", "-Xclang", "-packed-fp32-ops", "-Wno-unused-command-line-argument"]
# Extra compiler arguments (whitespace-separated), e.g. a different loop shape for an ablation run:
#   ATTN_HIPCC_EXTRA='-DATTN_D128_SHAPE=64,attn::LoopShape<8>' python exact_attention_76_amd/build.py
# (load_library() then loads that library only while ATTN_HIPCC_EXTRA holds the same arguments)
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


def source_record() -> dict:
    """sha256 of every file the library is compiled from, and the extra compiler arguments."""
    files = sorted(f for f in os.listdir(CSRC) if f.endswith((".hip", ".h")))
    rec = {f"csrc/{f}": hashlib.sha256(open(os.path.join(CSRC, f), "rb").read()).hexdigest() for f in files}
    rec["include/attn.h"] = hashlib.sha256(open(os.path.join(INCLUDE, "attn.h"), "rb").read()).hexdigest()
    return {"sources": rec, "extra_flags": os.environ.get("ATTN_HIPCC_EXTRA", "")}


def build() -> str:
    """Compile every source (in parallel), link libattn.so in the package directory and write
    its source record; returns the path of libattn.so."""
    os.makedirs(OBJ_DIR, exist_ok=True)
    record = source_record()
    with concurrent.futures.ThreadPoolExecutor(max_workers=len(SOURCES)) as ex:
        objs = list(ex.map(_compile, SOURCES))
    _link(objs, LIB)
    tmp = RECORD + ".tmp"
    with open(tmp, "w") as f:
        json.dump(record, f, indent=1, sort_keys=True)
    os.replace(tmp, RECORD)
    return LIB


if __name__ == "__main__":
    print(build())
