#!/usr/bin/env python3
"""Benchmark of the fused attention forward pass on one MI355X.

One step = one attn_fwd call over the whole workload (inputs already resident in HBM).
Workload: non-causal multi-head attention, bf16, B=1, N=16384, H=16, d=128 -- the longest
point of the B*N = 16384-token sweep (the pages quote their d=128 non-causal figure at 16k).

Metric (FlashAttention-3 digest, section 7.1): TFLOPs/s with FLOPs = 4 * B * H * N^2 * d
(halved when causal), and the fraction of MI355X dense bf16 MFMA peak.

Prints ONE JSON line with, besides the contract fields,
  roofline     -- the attention kernel's algorithmic FLOPs per launch over its mean launch
                  time (HIP events on the stream the kernel runs on) against the bf16 peak;
  cpu_baseline -- the fp64 CPU oracle timed on a bounded sample of query rows of the same
                  workload, as attention-FLOP throughput.
"""
from __future__ import annotations

import argparse
import json
import os
import sys
import time

import numpy as np

ROOT = os.path.dirname(os.path.abspath(__file__))
sys.path.insert(0, ROOT)

PEAK_BF16_TFLOPS = 2516.6  # 256 CU x 4096 dense bf16 FLOP/clk/CU x 2.4 GHz
WORKLOAD = dict(name="mha_n16384_b1_h16_d128", B=1, N=16384, H=16, d=128, causal=False, seed=2)
# HBM-side bytes per launch of the attention kernel from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE,
# scaled by the counters of a copy kernel of known size (profiles/fwd_bf16_d128_n16384_traffic.md).
# Valid only for the kernel source they were taken on; any other version reports null.
MEASURED_TRAFFIC = {"kernel_source": "exact_attention_76_amd/csrc/attn_fwd.hip",
                    "sha256_prefix": "21e9df9fc4856c3e", "bytes": 403843800}


def measured_traffic():
    import hashlib

    path = os.path.join(ROOT, MEASURED_TRAFFIC["kernel_source"])
    try:
        digest = hashlib.sha256(open(path, "rb").read()).hexdigest()
    except OSError:
        return None
    return MEASURED_TRAFFIC["bytes"] if digest.startswith(MEASURED_TRAFFIC["sha256_prefix"]) else None


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=50)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--cpu-seconds", type=float, default=12.0, help="target oracle time")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before timing, run one elementwise copy (negation) of this many MiB, so that "
                         "profiler byte counters can be scaled against a kernel of known traffic")
    return ap.parse_args()


def cpu_baseline(inp, target_s: float) -> dict:
    """Time the fp64 oracle on successive chunks of query rows until about target_s elapse."""
    import oracle

    q, k, v = (oracle.widen(getattr(inp, n), inp.dtype) for n in "qkv")
    rng = np.random.default_rng(123)
    T = inp.B * inp.N
    rows = 0
    flops = 0.0
    chunk = 1024
    t0 = time.perf_counter()
    while True:
        heads = rng.integers(0, inp.Hq, chunk)
        tokens = rng.integers(0, T, chunk)
        oracle.attention_rows(q, k, v, heads, tokens, causal=inp.causal, alpha=inp.alpha)
        rows += chunk
        keys = (tokens % inp.N + 1) if inp.causal else np.full(chunk, inp.N)
        flops += float(np.sum(4.0 * keys * inp.d))
        el = time.perf_counter() - t0
        if el >= target_s or el >= 30.0:
            break
    return {"value": flops / el / 1e12, "unit": "TFLOP/s", "cores": oracle.num_threads(),
            "kind": "oracle",
            "sample": f"{rows} random (head, query) rows of the same workload, all keys each, fp64, "
                      f"{el:.1f} s"}


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); every workload here fits one "
              "MI355X and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import torch

    import exact_attention_76_amd as ea
    import seeded_inputs as si

    w = WORKLOAD
    inp = si.dense_inputs(w["B"], w["N"], w["H"], w["d"], causal=w["causal"], seed=w["seed"])
    dev = torch.device("cuda:0")
    q, k, v = (torch.from_numpy(getattr(inp, n).view(np.int16)).view(torch.bfloat16).to(dev) for n in "qkv")
    o = torch.empty_like(q)
    lse = torch.empty((w["B"], w["H"], w["N"]), dtype=torch.float32, device=dev)
    stream = torch.cuda.Stream(device=dev)  # default priority
    flops = inp.flops()

    def step():
        ea.attn_fwd(q, k, v, o, lse, causal=w["causal"], alpha=inp.alpha, stream=stream)

    if args.calibration_copy_mib:
        n_el = args.calibration_copy_mib * (1 << 20) // 2
        src = torch.ones(n_el, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)  # reads and writes exactly calibration_copy_mib MiB each
        torch.cuda.synchronize()
        del src, dst
    torch.cuda.synchronize()
    with torch.cuda.stream(stream):
        for _ in range(args.warmup):
            step()
    torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(args.steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = time.perf_counter() - t0
    ms_gpu = ev0.elapsed_time(ev1) / args.steps
    ms_wall = wall * 1e3 / args.steps
    tflops = flops / (ms_wall * 1e-3) / 1e12
    achieved = flops / (ms_gpu * 1e-3) / 1e12

    roofline = {"bound": "mfma", "achieved": round(achieved, 2), "peak": PEAK_BF16_TFLOPS, "unit": "TFLOP/s",
                "frac": round(achieved / PEAK_BF16_TFLOPS, 4),
                "traffic": measured_traffic()}
    cpu = None
    if not args.no_cpu_baseline:
        cpu = cpu_baseline(inp, args.cpu_seconds)
        cpu["value"] = float(f"{cpu['value']:.4g}")

    line = {
        "metric": "attention fwd TFLOPs/s (4\u00b7B\u00b7H\u00b7N\u00b2\u00b7d, \u00bd if causal) and % of MI355X MFMA peak",
        "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_wall, 4), "higher_is_better": True,
        "scaling": "weak", "vs_baseline": None, "dtype": "bf16", "data": "synthetic",
        "config": {"workload": w["name"], "B": w["B"], "N": w["N"], "H": w["H"], "d": w["d"],
                   "causal": w["causal"], "global_batch": w["B"], "seq_len": w["N"],
                   "pct_of_peak": round(100 * tflops / PEAK_BF16_TFLOPS, 2), "parallelism": "single GPU"},
        "roofline": roofline,
        "cpu_baseline": cpu,
    }
    print(json.dumps(line), flush=True)


if __name__ == "__main__":
    main()
