#!/usr/bin/env python3
"""Benchmark of the fused attention forward pass on one MI355X.

One step = one attn_fwd call over the whole workload, inputs already resident in HBM.  Each
workload runs at least --warmup untimed steps, and keeps warming up until --warmup-seconds
(0.2 s) have passed, so that the timed steps run at the clock the chip settles at under load.
Default workload (the headline line): non-causal multi-head attention, bf16, B=1, N=16384,
H=16, d=128 -- the longest point of the B*N = 16384-token sweep (the pages quote their d=128
non-causal figure at 16k); the line's config also carries every point of that sweep and the
sweep's aggregate (total FLOPs over total time).  ``--workload`` selects the other measured configurations:

  sweep   bf16 non-causal d=128 H=16, N in 512..16384 with B*N = 16384 (one line per N)
  causal  bf16 causal B=2 H=16 N=8192, d in 64/128/256 (one line per d)
  varlen  bf16 causal GQA (Hq=32, Hkv=8, d=128), 8 packed sequences of 256..8192 tokens
  fp8     e4m3 non-causal B=2 H=16 N=8192 d=128 on pre-quantised inputs; the FP8 pre-pass
          (Hadamard rotation + block quantisation, HBM-bound) is timed separately
  fp8_causal  the same kernel causal, on the bf16 causal d=128 workload's inputs
  fp8_varlen  the same kernel on the packed causal GQA workload's inputs
  bwd     backward pass (attn_bwd: D pre-pass, dK/dV, dQ) on the headline inputs (B=1 N=16384,
          non-causal) and the causal d=128 inputs (B=2 N=8192); FLOPs = 2.5 x the forward's
  window  causal sliding window of 4096 keys, B=1 N=16384 H=16 d=128 (the headline's inputs), bf16
          then e4m3; FLOPs count the visible pairs, n^2/2 - (n-W)^2/2 per head

Metric (FlashAttention-3 digest, section 7.1): TFLOPs/s with FLOPs = 4 * B * H * N^2 * d
(halved when causal; summed per sequence for packed inputs), and the fraction of MI355X dense
MFMA peak (bf16 2516.6, fp8 5033.2 TFLOP/s at 2.4 GHz, 256 CUs).

Each line carries
  roofline     -- algorithmic FLOPs per launch over the kernel's mean launch time, measured
                  with HIP events on the stream the kernel runs on, against the dtype's peak;
  cpu_baseline -- (headline only) the fp64 CPU oracle timed on a bounded sample of query rows
                  of the same workload, as attention-FLOP throughput, on all host cores; with
                  per_config (the same for every other workload) and one_core (the smallest
                  workload and the N=4096 sweep point on one core);
and, in config, the median and best single launch from a second pass of the same K launches
with an event pair around each (after the timed region, so it does not perturb it), and sclk:
the graphics clock the power-management firmware reports while the same launch runs back to
back for 2.5 s after the timed region, with the dense peak recomputed at that clock.

The default line also carries, in config.workloads, every other workload timed the same way
(the smallest one, the causal head dims, the packed causal GQA workload, FP8 attention
with its pre-pass and where it stands against the FP8 accuracy bar, and the backward pass on
the headline and causal d=128 inputs), and config.targets: the bf16 and FP8 fractions of peak
against their goals.
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

METRIC = "attention fwd TFLOPs/s (4·B·H·N²·d, ½ if causal) and % of MI355X MFMA peak"
PEAK = {"bf16": 2516.6, "fp8": 5033.2}  # dense MFMA TFLOP/s: 256 CU x (4096 | 8192) FLOP/clk x 2.4 GHz
HBM_PEAK_GBS = 8000.0
# HBM-side bytes per launch from rocprofv3 --pmc FETCH_SIZE / WRITE_SIZE, each scaled by what the
# same counter reads for a copy kernel of known size (profiles/*_counters.md).  An entry is valid
# only for the kernel sources it was taken on (sha256 prefix of each file); any other version
# reports null.
_DEC = "exact_attention_76_amd/csrc/decompose.h"
_T16 = "exact_attention_76_amd/csrc/tile16.h"
MEASURED_TRAFFIC = {
    "bf16_mha16k": {"sources": {"exact_attention_76_amd/csrc/attn_fwd.hip": "a5caee0bd4413070",
                                _DEC: "2521a203b68b3442", _T16: "91339639cbec1225"},
                    "bytes": 403968001},
    "fp8_attention": {"sources": {"exact_attention_76_amd/csrc/fp8.hip": "42bf6866be33abb5",
                                  _DEC: "2521a203b68b3442"}, "bytes": 185858065},
    "fp8_prepare": {"sources": {"exact_attention_76_amd/csrc/fp8.hip": "42bf6866be33abb5"},
                    "bytes": 302757444},
}


def measured_traffic(key):
    import hashlib

    entry = MEASURED_TRAFFIC[key]
    for rel, prefix in entry["sources"].items():
        try:
            digest = hashlib.sha256(open(os.path.join(ROOT, rel), "rb").read()).hexdigest()
        except OSError:
            return None
        if not digest.startswith(prefix):
            return None
    return entry["bytes"]


def parse():
    ap = argparse.ArgumentParser()
    ap.add_argument("--gpus", type=int, default=1)
    ap.add_argument("--steps", type=int, default=100)
    ap.add_argument("--warmup", type=int, default=20)
    ap.add_argument("--warmup-seconds", type=float, default=0.2,
                    help="keep warming up (in rounds of --warmup steps) until this much time has passed; "
                         "0 gives exactly --warmup steps, e.g. for a fixed dispatch count under a profiler")
    ap.add_argument("--workload", default="mha16k", choices=["mha16k", "sweep", "causal", "varlen", "fp8", "fp8_causal",
                                                              "fp8_varlen", "window", "bwd"])
    ap.add_argument("--config", default=None,
                    help="with --workload sweep or causal: run only this configuration (e.g. mha_n512_b32_h16_d128), "
                         "for profiling one kernel instance")
    ap.add_argument("--no-cpu-baseline", action="store_true", help="skip the oracle timing leg")
    ap.add_argument("--no-clock", action="store_true",
                    help="skip the sustained-load clock reading (2.5 s of extra launches), e.g. under a profiler")
    ap.add_argument("--cpu-seconds", type=float, default=10.0, help="target oracle time of the headline baseline")
    ap.add_argument("--oracle-seconds", type=float, default=1.0,
                    help="target oracle time of each other workload's figure (default run)")
    ap.add_argument("--calibration-copy-mib", type=int, default=0,
                    help="before timing, run one elementwise copy (negation) of this many MiB, so that "
                         "profiler byte counters can be scaled against a kernel of known traffic")
    return ap.parse_args()


def cpu_baseline(inp, target_s: float, threads: int | None = None) -> dict:
    """Time the fp64 oracle on successive chunks of random (head, query) rows of the workload
    until about target_s elapse (every visible key of each row); with ``threads``, on that many
    OpenMP threads.  Returns attention-FLOP throughput (4 d FLOP per visible key)."""
    import oracle

    q, k, v = (oracle.widen(getattr(inp, n), inp.dtype) for n in "qkv")
    rng = np.random.default_rng(123)
    cu = inp.cu_seqlens.astype(np.int64) if inp.cu_seqlens is not None else np.arange(inp.B + 1) * inp.N
    T = int(cu[-1])
    rows = 0
    flops = 0.0
    chunk = 1024
    default_threads = oracle.num_threads()
    if threads is not None:
        oracle.set_num_threads(threads)
    try:
        t0 = time.perf_counter()
        while True:
            heads = rng.integers(0, inp.Hq, chunk)
            tokens = rng.integers(0, T, chunk)
            oracle.attention_rows(q, k, v, heads, tokens, causal=inp.causal, alpha=inp.alpha,
                                  cu_seqlens=inp.cu_seqlens, window=inp.window)
            rows += chunk
            seq = np.searchsorted(cu, tokens, side="right") - 1
            i = tokens - cu[seq]
            keys = (i + 1) if inp.causal else (cu[seq + 1] - cu[seq])
            if inp.window:
                keys = np.minimum(keys, inp.window)
            flops += float(np.sum(4.0 * keys * inp.d))
            el = time.perf_counter() - t0
            if el >= target_s or el >= 30.0:
                break
        used = oracle.num_threads()
    finally:
        oracle.set_num_threads(default_threads)
    return {"value": float(f"{flops / el / 1e12:.4g}"), "unit": "TFLOP/s", "cores": used,
            "kind": "oracle", "cpu_model": cpu_model(),
            "sample": f"{rows} random (head, query) rows of the same workload, all keys each, fp64, {el:.1f} s"}


def timed(step, stream, steps, warmup, min_seconds=0.0):
    """At least W untimed steps, continued until ``min_seconds`` of them have run (the clock
    needs that long under load to settle; a short step's 20 warmups take a few ms), then K
    steps between two synchronisations.  Returns (wall ms per step, event ms per step measured
    on ``stream``)."""
    import torch

    torch.cuda.synchronize()
    t0 = time.perf_counter()
    for _ in range(warmup):
        step()
    torch.cuda.synchronize()
    while time.perf_counter() - t0 < min_seconds:
        for _ in range(max(1, warmup)):
            step()
        torch.cuda.synchronize()
    ev0, ev1 = torch.cuda.Event(enable_timing=True), torch.cuda.Event(enable_timing=True)
    t0 = time.perf_counter()
    ev0.record(stream)
    for _ in range(steps):
        step()
    ev1.record(stream)
    torch.cuda.synchronize()
    wall = (time.perf_counter() - t0) * 1e3 / steps
    return wall, ev0.elapsed_time(ev1) / steps


def per_launch(step, stream, steps):
    """After the timed region: the same launches again, each between two events on ``stream``.
    Returns (median ms, min ms) per launch."""
    import torch

    evs = [torch.cuda.Event(enable_timing=True) for _ in range(steps + 1)]
    torch.cuda.synchronize()
    evs[0].record(stream)
    for i in range(steps):
        step()
        evs[i + 1].record(stream)
    torch.cuda.synchronize()
    ms = np.array([evs[i].elapsed_time(evs[i + 1]) for i in range(steps)])
    return float(np.median(ms)), float(ms.min())


def cpu_model() -> str:
    try:
        for line_ in open("/proc/cpuinfo"):
            if line_.startswith("model name"):
                return line_.split(":", 1)[1].strip()
    except OSError:
        pass
    return "unknown"


def sustained_clock(step, seconds: float = 2.5, settle: float = 1.2):
    """The graphics clock and socket power while ``step`` runs back to back for ``seconds``.

    Source: amdsmi gpu_metrics, current_gfxclk of each XCD (an average the power-management
    firmware refreshes about once a second) and current socket power.  Readings taken in the
    first ``settle`` seconds still cover time before the load began and are dropped.  These are
    reads of the management interface only; nothing else is launched.  Returns None when the
    interface is unavailable."""
    import threading

    import torch

    try:
        import amdsmi

        amdsmi.amdsmi_init()
        handles = amdsmi.amdsmi_get_processor_handles()
        handle = handles[0] if len(handles) == 1 else None
        if handle is None:
            bus = getattr(torch.cuda.get_device_properties(torch.cuda.current_device()), "pci_bus_id", None)
            for h in handles:
                if bus is not None and int(amdsmi.amdsmi_get_gpu_device_bdf(h).split(":")[1], 16) == int(bus):
                    handle = h
        if handle is None:
            return None
    except Exception:  # noqa: BLE001 -- no management interface: report no clock
        return None
    samples, stop = [], threading.Event()

    def poll():
        while not stop.is_set():
            try:
                m = amdsmi.amdsmi_get_gpu_metrics_info(handle)
            except Exception:  # noqa: BLE001
                return
            clks = m.get("current_gfxclks")
            vals = [x for x in clks if isinstance(x, (int, float)) and 0 < x < 10000] if isinstance(clks, list) else []
            pw = m.get("current_socket_power")
            samples.append((time.perf_counter(), sum(vals) / len(vals) if vals else None,
                            pw if isinstance(pw, (int, float)) and 0 < pw < 100000 else None))
            stop.wait(0.05)

    th = threading.Thread(target=poll, daemon=True)
    t0 = time.perf_counter()
    th.start()
    while time.perf_counter() - t0 < seconds:
        for _ in range(8):
            step()
        torch.cuda.synchronize()
    stop.set()
    th.join()
    clk = [c for t, c, _ in samples if t - t0 >= settle and c is not None]
    pw = [p for t, _, p in samples if t - t0 >= settle and p is not None]
    if not clk:
        return None
    return {"mean_mhz": round(float(np.mean(clk)), 1), "min_mhz": round(float(np.min(clk)), 1),
            "max_mhz": round(float(np.max(clk)), 1), "socket_power_w": round(float(np.mean(pw)), 1) if pw else None,
            "samples": len(clk), "window_s": seconds - settle,
            "source": "amdsmi gpu_metrics current_gfxclk (firmware average per XCD, refreshed about once a "
                      "second), sampled while the same launch ran back to back after the timed region"}


def to_dev(bits, dtype, dev):
    import torch

    t = torch.from_numpy(bits.view(np.int16))
    return t.view(torch.bfloat16 if dtype == "bf16" else torch.float16).to(dev)


def line(args, name, inp, flops, ms_wall, ms_gpu, dtype, extra=None, traffic=None, cpu=None, launches=None):
    peak = PEAK[dtype]
    tflops = flops / (ms_wall * 1e-3) / 1e12
    achieved = flops / (ms_gpu * 1e-3) / 1e12
    cfg = {"workload": name, "B": inp.B, "N": inp.N, "Hq": inp.Hq, "Hkv": inp.Hkv, "d": inp.d,
           "causal": inp.causal, "varlen": inp.cu_seqlens is not None, "tokens": inp.total_tokens,
           "flops_per_step": flops, "pct_of_peak": round(100 * tflops / peak, 2), "parallelism": "single GPU",
           "warmup_min_seconds": args.warmup_seconds}
    if inp.window:
        cfg["window"] = inp.window
    if launches is not None:
        med, best = launches
        cfg.update({"ms_event_mean": round(ms_gpu, 4), "ms_launch_median": round(med, 4), "ms_launch_min": round(best, 4),
                    "tflops_launch_median": round(flops / (med * 1e-3) / 1e12, 2),
                    "tflops_launch_best": round(flops / (best * 1e-3) / 1e12, 2)})
    if extra:
        cfg.update(extra)
    clk = cfg.get("sclk")
    if clk:
        # the nominal peak assumes 2.4 GHz; the same units at the observed mean clock
        at_clk = peak * clk["mean_mhz"] / 2400.0
        cfg["peak_at_observed_sclk"] = round(at_clk, 1)
        cfg["pct_of_peak_at_observed_sclk"] = round(100 * achieved / at_clk, 2)
    return {
        "metric": METRIC, "value": round(tflops, 2), "unit": "TFLOP/s", "n_gpus": 1, "steps": args.steps,
        "warmup": args.warmup, "ms_per_step": round(ms_wall, 4), "higher_is_better": True, "scaling": "weak",
        "vs_baseline": None, "dtype": dtype, "data": "synthetic", "config": cfg,
        "roofline": {"bound": "mfma", "achieved": round(achieved, 2), "peak": peak, "unit": "TFLOP/s",
                     "frac": round(achieved / peak, 4), "traffic": traffic},
        "cpu_baseline": cpu,
    }


def run_16bit(args, name, inp, dev, stream, traffic=None, cpu=False, oracle_s=0.0, clock=False):
    import torch

    import exact_attention_76_amd as ea

    q, k, v = (to_dev(getattr(inp, n), inp.dtype, dev) for n in "qkv")
    o = torch.empty_like(q)
    if inp.cu_seqlens is None:
        lse = torch.empty((inp.B, inp.Hq, inp.N), dtype=torch.float32, device=dev)
        cu = None
    else:
        lse = torch.empty((inp.Hq, inp.total_tokens), dtype=torch.float32, device=dev)
        cu = torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev)

    def step():
        if inp.window:
            ea.attn_fwd_window(q, k, v, o, lse, window=inp.window, alpha=inp.alpha, cu_seqlens=cu,
                               max_seqlen=inp.N if cu is not None else None, stream=stream)
        else:
            ea.attn_fwd(q, k, v, o, lse, causal=inp.causal, alpha=inp.alpha, cu_seqlens=cu,
                        max_seqlen=inp.N if cu is not None else None, stream=stream)

    ms_wall, ms_gpu = timed(step, stream, args.steps, args.warmup, args.warmup_seconds)
    launches = per_launch(step, stream, args.steps)
    cpu_res = cpu_baseline(inp, args.cpu_seconds) if cpu and not args.no_cpu_baseline else None
    extra = {"sclk": sustained_clock(step)} if clock and not args.no_clock else {}
    if oracle_s > 0 and not args.no_cpu_baseline:
        extra["oracle"] = cpu_baseline(inp, oracle_s)
    return line(args, name, inp, inp.flops(), ms_wall, ms_gpu, inp.dtype, traffic=traffic, cpu=cpu_res,
                launches=launches, extra=extra)


# FP8 workloads: name of the line -> the seeded bf16 inputs it quantises
FP8_WORKLOADS = {"fp8": "fp8_b2_h16_n8192_d128", "fp8_causal": "causal_b2_h16_n8192_d128",
                 "fp8_varlen": "gqa_varlen_causal_hq32_hkv8_d128"}
WINDOW = 4096  # keys of the sliding-window workload


def window_inputs():
    import seeded_inputs as si

    inp = si.CONFIGS["mha_n16384_b1_h16_d128"]()
    inp.causal, inp.window = True, WINDOW
    return inp


def run_fp8(args, dev, stream, workload="fp8", inp=None, oracle_s=0.0, clock=False):
    import torch

    import exact_attention_76_amd as ea
    import seeded_inputs as si

    src = FP8_WORKLOADS.get(workload, workload)
    inp = si.CONFIGS[src]() if inp is None else inp
    q, k, v = (to_dev(getattr(inp, n), "bf16", dev) for n in "qkv")
    signs = torch.from_numpy(si.hadamard_signs(inp.d)).to(dev)
    packed = {}
    if inp.cu_seqlens is not None:
        packed = dict(cu_seqlens=torch.from_numpy(inp.cu_seqlens.astype(np.int32)).to(dev), max_seqlen=inp.N)
    q8, k8, v8, qs, ks, vs = ea.fp8_prepare(q, k, v, hadamard_signs=signs, stream=stream, **packed)
    o = torch.empty(q.shape, dtype=torch.bfloat16, device=dev)
    lse_shape = (inp.B, inp.Hq, inp.N) if not packed else (inp.Hq, inp.total_tokens)
    lse = torch.empty(lse_shape, dtype=torch.float32, device=dev)

    def attn():
        kw = dict(alpha=inp.alpha, q_scale=qs, k_scale=ks, v_scale=vs, stream=stream, **packed)
        if inp.window:
            ea.attn_fwd_window(q8, k8, v8, o, lse, window=inp.window, **kw)
        else:
            ea.attn_fwd(q8, k8, v8, o, lse, causal=inp.causal, **kw)

    def prep():
        ea.attn_fp8_prepare_ex(q, k, v, q8, k8, v8, qs, ks, vs, hadamard_signs=signs, stream=stream, **packed)

    ms_wall, ms_gpu = timed(attn, stream, args.steps, args.warmup, args.warmup_seconds)
    launches = per_launch(attn, stream, args.steps)
    clk = sustained_clock(attn) if clock and not args.no_clock else None
    pw, pg = timed(prep, stream, args.steps, args.warmup, args.warmup_seconds)
    elems = q.numel() + k.numel() + v.numel()
    prep_bytes = 2 * elems + elems + (qs.numel() + ks.numel() + vs.numel()) * 4 + inp.d
    rope_extra = {}
    if workload == "fp8" and inp.window == 0:
        # the same pre-pass fused with a rotary embedding (fp32 tables [N, d/2])
        cos, sin = (torch.from_numpy(t).to(dev) for t in si.rope_tables(inp.N, inp.d))

        def rope_prep():
            ea.attn_fp8_prepare_ex(q, k, v, q8, k8, v8, qs, ks, vs, hadamard_signs=signs, rope_cos=cos, rope_sin=sin,
                                   stream=stream)

        rw, rg = timed(rope_prep, stream, args.steps, args.warmup, args.warmup_seconds)
        rbytes = prep_bytes + 2 * cos.numel() * 4
        rope_extra = {"rope_prepare_ms": round(rw, 4),
                      "rope_prepare_roofline": {"bound": "hbm", "achieved": round(rbytes / (rg * 1e-3) / 1e9, 1),
                                                "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                                "frac": round(rbytes / (rg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                                "bytes_per_launch": rbytes},
                      "rope_unfused_extra_bytes": 4 * (q.numel() + k.numel())}
    extra = {"attention_only": True, "hadamard": True, "inputs_from": src, "sclk": clk,
             "prepare_ms": round(pw, 4),
             "prepare_roofline": {"bound": "hbm", "achieved": round(prep_bytes / (pg * 1e-3) / 1e9, 1),
                                  "peak": HBM_PEAK_GBS, "unit": "GB/s",
                                  "frac": round(prep_bytes / (pg * 1e-3) / 1e9 / HBM_PEAK_GBS, 4),
                                  "traffic": measured_traffic("fp8_prepare") if workload == "fp8" else None,
                                  "bytes_per_launch": prep_bytes},
             "prepare_plus_attention_tflops": round(inp.flops() / ((pw + ms_wall) * 1e-3) / 1e12, 2), **rope_extra}
    if workload == "fp8" and inp.window == 0:
        extra["accuracy"] = fp8_accuracy_note()
    if oracle_s > 0 and not args.no_cpu_baseline:
        extra["oracle"] = cpu_baseline(inp, oracle_s)
    name = "fp8_b2_h16_n8192_d128" if workload == "fp8" else f"fp8_{src}"
    if inp.window:
        name = f"fp8_window{inp.window}_b1_h16_n16384_d128"
    return line(args, name, inp, inp.flops(), ms_wall, ms_gpu, "fp8", extra=extra,
                traffic=measured_traffic("fp8_attention") if workload == "fp8" else None, launches=launches)


def fp8_accuracy_note() -> dict:
    """Where the FP8 workload stands against the FP8 bar (O RMSE <= 3e-2 against fp64 on the
    unquantised inputs), from the floor the tests pin on the CPU from the oracle alone."""
    floor = None
    try:
        for line_ in open(os.path.join(ROOT, "tests", "golden", "fp8_quantisation_floors.txt")):
            if line_.startswith("c5_shared_channels "):
                floor = float(line_.split()[1])
    except OSError:
        pass
    return {"bar_rmse": 3e-2, "quantisation_floor_rmse": floor,
            "reading": "two x20 outlier channels shared by Q, K and V: quantising the inputs alone "
                       "(exact attention on the e4m3-dequantised inputs) already costs the floor, above "
                       "the bar, so the bar is not met on this reading (the kernel measures about 0.036 "
                       "and is held to the floor + 2e-3); with independent outlier channels per tensor the "
                       "floor is 0.011 and the kernel meets the bar",
            "floor_source": "tests/golden/fp8_quantisation_floors.txt (oracle only)"}


def summary(r: dict) -> dict:
    """The figures of one bench line that the headline line carries for it."""
    c = r["config"]
    out = {"tflops": r["value"], "pct_of_peak": c["pct_of_peak"], "dtype": r["dtype"],
           "ms_per_step": r["ms_per_step"], "roofline_frac": r["roofline"]["frac"],
           "tflops_launch_median": c.get("tflops_launch_median")}
    for key in ("peak_at_observed_sclk", "pct_of_peak_at_observed_sclk"):
        if key in c:
            out[key] = c[key]
    if c.get("sclk"):
        out["sclk_mean_mhz"] = c["sclk"]["mean_mhz"]
    if c.get("oracle"):
        out["oracle_tflops"] = c["oracle"]["value"]
        out["oracle_cores"] = c["oracle"]["cores"]
    for key in ("prepare_ms", "prepare_roofline", "prepare_plus_attention_tflops", "accuracy"):
        if key in c:
            out[key] = c[key]
    return out


def run_bwd(args, name, inp, dev, stream):
    """The backward pass on inputs resident in HBM (Q, K, V, O, L from the forward, dO)."""
    import torch

    import exact_attention_76_amd as ea
    import seeded_inputs as si

    q, k, v = (to_dev(getattr(inp, n), inp.dtype, dev) for n in "qkv")
    do = to_dev(si.output_gradient(inp, 9), inp.dtype, dev)
    o, lse = ea.attention(q, k, v, causal=inp.causal, alpha=inp.alpha, stream=stream)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(inp.B * inp.Hq * inp.N, dtype=torch.float32, device=dev)

    def step():
        ea.attn_bwd(q, k, v, o, lse, do, dq, dk, dv, ws, causal=inp.causal, alpha=inp.alpha, stream=stream)

    ms_wall, ms_gpu = timed(step, stream, args.steps, args.warmup, args.warmup_seconds)
    launches = per_launch(step, stream, args.steps)
    return line(args, name, inp, 2.5 * inp.flops(), ms_wall, ms_gpu, inp.dtype, launches=launches,
                extra={"pass": "backward", "flops_rule": "2.5 x forward (five products)"})


def main():
    args = parse()
    if args.gpus != 1:
        print(f"bench.py runs on one GPU only (asked for {args.gpus}); every workload here fits one "
              "MI355X and no multi-GPU path is built", file=sys.stderr)
        sys.exit(2)

    import torch

    import seeded_inputs as si

    dev = torch.device("cuda:0")
    stream = torch.cuda.Stream(device=dev)  # default priority
    if args.calibration_copy_mib:
        n_el = args.calibration_copy_mib * (1 << 20) // 2
        src = torch.ones(n_el, dtype=torch.bfloat16, device=dev)
        dst = torch.empty_like(src)
        torch.neg(src, out=dst)  # reads and writes exactly calibration_copy_mib MiB each
        torch.cuda.synchronize()
        del src, dst

    with torch.cuda.stream(stream):
        if args.workload == "mha16k":
            name = "mha_n16384_b1_h16_d128"
            head = run_16bit(args, name, si.CONFIGS[name](), dev, stream, traffic=measured_traffic("bf16_mha16k"),
                             cpu=True, oracle_s=args.oracle_seconds, clock=True)
            # the rest of the B*N = 16384 sweep this figure belongs to, attached for context
            sweep, flops, ms = {}, 0.0, 0.0
            workloads = {}
            for n in si.CONFIGS:
                if not n.startswith("mha_n"):
                    continue
                r = head if n == name else run_16bit(args, n, si.CONFIGS[n](), dev, stream,
                                                      oracle_s=args.oracle_seconds)
                sweep[f"N={r['config']['N']}"] = r["value"]
                workloads[n] = summary(r)
                flops += r["config"]["flops_per_step"]
                ms += r["ms_per_step"]
            head["config"]["sweep_tflops"] = sweep
            head["config"]["sweep_aggregate_tflops"] = round(flops / (ms * 1e-3) / 1e12, 2)
            # every other workload, timed the same way: the smallest (launch-bound), the causal
            # head dims, the packed causal GQA workload and FP8 (attention and pre-pass)
            for n in ["mha_b1_h2_n128_d64"] + [c for c in si.CONFIGS if c.startswith("causal")] + \
                     ["gqa_varlen_causal_hq32_hkv8_d128"]:
                workloads[n] = summary(run_16bit(args, n, si.CONFIGS[n](), dev, stream, oracle_s=args.oracle_seconds))
            r8 = run_fp8(args, dev, stream, "fp8", oracle_s=args.oracle_seconds, clock=True)
            workloads["fp8_b2_h16_n8192_d128"] = summary(r8)
            # the backward pass on the headline and the causal d=128 inputs (2.5 x forward FLOPs)
            for n in ("mha_n16384_b1_h16_d128", "causal_b2_h16_n8192_d128"):
                workloads["bwd_" + n] = summary(run_bwd(args, "bwd_" + n, si.CONFIGS[n](), dev, stream))
            head["config"]["workloads"] = workloads
            head["config"]["targets"] = {
                "bf16_headline_pct_of_peak": {"target": 60.0, "measured": head["config"]["pct_of_peak"]},
                "fp8_pct_of_peak": {"target": 45.0, "measured": workloads["fp8_b2_h16_n8192_d128"]["pct_of_peak"]}}
            if head["cpu_baseline"] is not None:
                cb = head["cpu_baseline"]
                cb["per_config"] = {n: {"tflops": w["oracle_tflops"], "cores": w["oracle_cores"]}
                                    for n, w in workloads.items() if "oracle_tflops" in w}
                # the same oracle on one core, for a per-core figure
                cb["one_core"] = {n: cpu_baseline(si.CONFIGS[n](), args.oracle_seconds * 2, threads=1)
                                  for n in ("mha_b1_h2_n128_d64", "mha_n4096_b4_h16_d128")}
            out = [head]
        elif args.workload == "sweep":
            out = [run_16bit(args, n, si.CONFIGS[n](), dev, stream, clock=True)
                   for n in si.CONFIGS if n.startswith("mha_n") and args.config in (None, n)]
        elif args.workload == "causal":
            out = [run_16bit(args, n, si.CONFIGS[n](), dev, stream, clock=True)
                   for n in si.CONFIGS if n.startswith("causal") and args.config in (None, n)]
        elif args.workload == "varlen":
            n = "gqa_varlen_causal_hq32_hkv8_d128"
            out = [run_16bit(args, n, si.CONFIGS[n](), dev, stream, clock=True)]
        elif args.workload in FP8_WORKLOADS:
            out = [run_fp8(args, dev, stream, args.workload, clock=True)]
        elif args.workload == "bwd":
            out = [run_bwd(args, "bwd_" + n, si.CONFIGS[n](), dev, stream)
                   for n in ("mha_n16384_b1_h16_d128", "causal_b2_h16_n8192_d128")]
        else:  # window
            out = [run_16bit(args, f"window{WINDOW}_b1_h16_n16384_d128", window_inputs(), dev, stream),
                   run_fp8(args, dev, stream, "mha_n16384_b1_h16_d128", inp=window_inputs())]
    for o in out:
        print(json.dumps(o), flush=True)


if __name__ == "__main__":
    main()
