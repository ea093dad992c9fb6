"""Shared helpers of the GPU tests: move seeded inputs to the device, run libattn, compare
with the oracle.  Importing this module does not touch the GPU."""
from __future__ import annotations

import sys

import numpy as np
import torch

import oracle
import seeded_inputs

# Tolerances on O and LSE against the fp64 oracle (bf16 and fp16 outputs).
TOL_MAX_ABS = 1e-2
TOL_RMSE = 2e-3
TOL_LSE = 1e-3
TOL_FP8_RMSE = 3e-2


def say(*args):
    """Name the case before a GPU step (flushed, so it survives a crash of the process)."""
    print("[case]", *args, file=sys.stderr, flush=True)


def torch_dtype(dtype: str):
    return {"bf16": torch.bfloat16, "fp16": torch.float16}[dtype]


def to_device(inp: seeded_inputs.AttnInputs):
    dt = torch_dtype(inp.dtype)
    q, k, v = (torch.from_numpy(getattr(inp, n).view(np.int16)).view(dt).cuda() for n in "qkv")
    cu = None if inp.cu_seqlens is None else torch.from_numpy(inp.cu_seqlens.astype(np.int32)).cuda()
    return q, k, v, cu


def attention_nan(q, k, v, *, causal=False, alpha=None, cu_seqlens=None, max_seqlen=None, window=None,
                  q_scale=None, k_scale=None, v_scale=None):
    """attn_fwd (or attn_fwd_window) into O and LSE pre-filled with NaN: a row that no workgroup
    writes stays NaN, so the tests' finiteness checks prove that every row was written."""
    import exact_attention_76_amd as ea

    out_dtype = torch.float16 if q.dtype == torch.float16 else torch.bfloat16
    o = torch.full(q.shape, float("nan"), dtype=out_dtype, device=q.device)
    lse_shape = (q.shape[0], q.shape[2], q.shape[1]) if cu_seqlens is None else (q.shape[1], q.shape[0])
    lse = torch.full(lse_shape, float("nan"), dtype=torch.float32, device=q.device)
    torch.cuda.synchronize()
    kw = dict(alpha=alpha, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, q_scale=q_scale, k_scale=k_scale,
              v_scale=v_scale)
    if window:
        ea.attn_fwd_window(q, k, v, o, lse, window=window, **kw)
    else:
        ea.attn_fwd(q, k, v, o, lse, causal=causal, **kw)
    return o, lse


def run_gpu(inp: seeded_inputs.AttnInputs):
    """libattn forward on the device; returns float64 numpy O (input layout) and LSE."""
    q, k, v, cu = to_device(inp)
    o, lse = attention_nan(q, k, v, causal=inp.causal, alpha=inp.alpha, cu_seqlens=cu,
                           max_seqlen=inp.N if cu is not None else None, window=inp.window or None)
    torch.cuda.synchronize()
    return o.double().cpu().numpy(), lse.double().cpu().numpy()


def widened(inp):
    return tuple(oracle.widen(getattr(inp, n), inp.dtype) for n in "qkv")


def oracle_full(inp):
    q, k, v = widened(inp)
    return oracle.attention(q, k, v, causal=inp.causal, alpha=inp.alpha, cu_seqlens=inp.cu_seqlens,
                            window=inp.window)


def sample_rows(inp, n: int, seed: int = 0):
    """Rows (head, packed token) to check at full size: the first and last token of every
    sequence plus uniformly drawn ones."""
    rng = np.random.default_rng(seed)
    cu = inp.cu_seqlens.astype(np.int64) if inp.cu_seqlens is not None else np.arange(inp.B + 1) * inp.N
    T = int(cu[-1])
    toks = [cu[:-1], cu[1:] - 1, rng.integers(0, T, n)]
    tokens = np.concatenate(toks)
    heads = rng.integers(0, inp.Hq, len(tokens))
    return heads, tokens


def coverage_rows(inp, br: int, whole_heads=None, seed: int = 0):
    """Rows (head, packed token) that cover a full-size launch: one query drawn from every
    (sequence, head, query block of br queries) -- so every workgroup of the grid has at least
    one checked row -- plus every token of the heads in ``whole_heads`` (default: the first and
    the last head, which sit on different XCDs and, with grouped heads, different KV groups)."""
    rng = np.random.default_rng(seed)
    cu = inp.cu_seqlens.astype(np.int64) if inp.cu_seqlens is not None else np.arange(inp.B + 1) * inp.N
    whole = (0, inp.Hq - 1) if whole_heads is None else whole_heads
    heads, tokens = [], []
    for b in range(len(cu) - 1):
        n = int(cu[b + 1] - cu[b])
        for q0 in range(0, n, br):
            cnt = min(br, n - q0)
            heads.append(np.arange(inp.Hq))
            tokens.append(cu[b] + q0 + rng.integers(0, cnt, inp.Hq))
    T = int(cu[-1])
    for h in whole:
        heads.append(np.full(T, h))
        tokens.append(np.arange(T))
    return np.concatenate(heads).astype(np.int64), np.concatenate(tokens).astype(np.int64)


def gpu_rows(inp, o_gpu, lse_gpu, heads, tokens):
    """Pick the sampled rows out of full GPU outputs."""
    if inp.cu_seqlens is None:
        T = inp.B * inp.N
        o = o_gpu.reshape(T, inp.Hq, inp.d)[tokens, heads]
        b, i = tokens // inp.N, tokens % inp.N
        lse = lse_gpu[b, heads, i]
    else:
        o = o_gpu[tokens, heads]
        lse = lse_gpu[heads, tokens]
    return o, lse


def half_ulp(x: np.ndarray, dtype: str) -> np.ndarray:
    """Half a unit in the last place of the output format at |x| (bf16: 8 significant bits,
    fp16: 11), i.e. the largest error of rounding the exact result to that format."""
    bits = {"bf16": 8, "fp16": 11}[dtype]
    ax = np.abs(np.asarray(x, dtype=np.float64))
    e = np.floor(np.log2(np.where(ax > 0, ax, 1.0)))
    if dtype == "fp16":
        e = np.maximum(e, -14.0)
    return np.where(ax > 0, 2.0 ** (e - bits), 0.0)


def metrics(o_test, o_ref, lse_test, lse_ref, dtype: str) -> dict:
    """Error measures against the fp64 oracle.  ``max_abs_excess`` is the largest error left
    after subtracting, element by element, the half ulp that rounding the exact O to the
    output format costs on its own (for |O| >= 4 half a bf16 ulp is 0.0156, more than the
    whole 1e-2 budget; this reading keeps 1e-2 as the bound on the kernel's own error)."""
    m = oracle.error_metrics(o_test, o_ref, lse_test, lse_ref)
    err = np.abs(np.asarray(o_test, dtype=np.float64) - np.asarray(o_ref, dtype=np.float64))
    m["max_abs_excess"] = float(np.max(err - half_ulp(o_ref, dtype))) if err.size else 0.0
    return m


def check(metrics: dict, *, max_abs=TOL_MAX_ABS, rmse=TOL_RMSE, lse=TOL_LSE, what=""):
    key = "max_abs_excess" if "max_abs_excess" in metrics else "max_abs"
    assert metrics[key] <= max_abs, f"{what}: O {key} {metrics[key]:.3e} > {max_abs} ({metrics})"
    assert metrics["rmse"] <= rmse, f"{what}: O RMSE {metrics['rmse']:.3e} > {rmse}"
    if "lse_max_abs" in metrics and lse is not None:
        assert metrics["lse_max_abs"] <= lse, f"{what}: LSE error {metrics['lse_max_abs']:.3e} > {lse}"
