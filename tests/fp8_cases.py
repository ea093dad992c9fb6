"""FP8 parity cases whose inputs alone already cost more than the FP8 bar (O RMSE <= 3e-2
against fp64 on the unquantised inputs): their outlier channels leave, after e4m3 block
quantisation, an error that exact attention on the dequantised inputs carries too -- the floor
any implementation of the method meets.  This module names each case's inputs and the rows the
GPU test checks, and computes the floor from the oracle alone (oracle/, the fp64 attention and
the e4m3 pre-pass emulation), so it can be pinned on the CPU (tests/test_fp8_floors.py,
tests/golden/fp8_quantisation_floors.txt) and the GPU tests gate the kernel against the stored
value, never against one recomputed from the kernel's own output.

The error measure is that of the FlashAttention-3 digest's section 3.5 / Table 3 (RMSE of O
against an fp64 reference on the unquantised inputs)."""
from __future__ import annotations

import os

import numpy as np

import oracle
import seeded_inputs as si
from oracle import fp8 as ofp8

FLOORS_FILE = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "fp8_quantisation_floors.txt")


def sample_rows(inp, n: int, seed: int):
    """The first and last token of every sequence plus n uniformly drawn (head, token) rows."""
    rng = np.random.default_rng(seed)
    cu = inp.cu_seqlens.astype(np.int64) if inp.cu_seqlens is not None else np.arange(inp.B + 1) * inp.N
    tokens = np.concatenate([cu[:-1], cu[1:] - 1, rng.integers(0, int(cu[-1]), n)])
    heads = rng.integers(0, inp.Hq, len(tokens))
    return heads, tokens


def all_rows(inp):
    T = inp.B * inp.N if inp.cu_seqlens is None else int(inp.cu_seqlens[-1])
    return np.repeat(np.arange(inp.Hq), T), np.tile(np.arange(T), inp.Hq)


VARLEN_SMALL = [1, 63, 64, 65, 200, 129, 300]


def varlen_small(causal: bool, seed: int):
    """Packed sequences of 1 .. 300 tokens (single-token, one-short, exact and one-over block
    sizes), 8 query heads on 2 KV heads, Q scaled by 3 so several block exponents occur."""
    inp = si.varlen_inputs(VARLEN_SMALL, 8, 2, 128, causal=causal, seed=seed)
    inp.q = si.f32_to_bf16_bits(si.bf16_bits_to_f32(inp.q) * np.float32(3.0))
    return inp


def case(name: str):
    """(inputs, Hadamard signs or None, heads, tokens, per-tensor scaling) of a pinned case."""
    signs = si.hadamard_signs(128, seed=55)
    if name in ("small_rotated", "small_unrotated"):
        inp = si.fp8_inputs(2, 300, 4, 128, seed=601, fraction=0.002)
        return (inp, signs if name == "small_rotated" else None, *all_rows(inp), False)
    if name == "c5_shared_channels":
        inp = si.CONFIGS["fp8_b2_h16_n8192_d128"]()
        return (inp, signs, *sample_rows(inp, 2048, seed=2), False)
    if name.startswith("varlen_small_"):
        _, _, mode, scaling = name.split("_")
        inp = varlen_small(mode == "causal", 612)
        return (inp, signs, *all_rows(inp), scaling == "tensor")
    raise KeyError(name)


CASES = ("small_rotated", "small_unrotated", "c5_shared_channels",
         "varlen_small_causal_block", "varlen_small_causal_tensor",
         "varlen_small_noncausal_block", "varlen_small_noncausal_tensor")


def quantisation_floor(inp, signs, heads, tokens, per_tensor=False) -> dict:
    """Error metrics of exact fp64 attention on the e4m3-dequantised inputs (the oracle's
    pre-pass: optional rotation, per-block or per-tensor power-of-two scales) against exact fp64
    attention on the unquantised inputs, over the given rows."""
    q, k, v = (oracle.bf16_to_f64(getattr(inp, n)) for n in "qkv")
    if inp.cu_seqlens is None:
        q8, k8, v8, qs, ks, vs = ofp8.fp8_prepare(q, k, v, signs, per_tensor=per_tensor)
        qd, kd, vd = ofp8.dequantize(q8, qs), ofp8.dequantize(k8, ks), ofp8.dequantize(v8, vs)
    else:
        q8, k8, v8, qs, ks, vs = ofp8.fp8_prepare_varlen(q, k, v, inp.cu_seqlens, inp.N, signs,
                                                          per_tensor=per_tensor)
        qd, kd, vd = (ofp8.dequantize_varlen(c, sc, inp.cu_seqlens) for c, sc in ((q8, qs), (k8, ks), (v8, vs)))
    kw = dict(causal=inp.causal, alpha=inp.alpha, cu_seqlens=inp.cu_seqlens)
    o_ref, l_ref = oracle.attention_rows(q, k, v, heads, tokens, **kw)
    o_dq, l_dq = oracle.attention_rows(qd, kd, vd, heads, tokens, **kw)
    return oracle.error_metrics(o_dq, o_ref, l_dq, l_ref)


def stored_floors() -> dict:
    """The pinned floors (O RMSE) from tests/golden/fp8_quantisation_floors.txt."""
    out = {}
    for line in open(FLOORS_FILE):
        line = line.strip()
        if line and not line.startswith("#"):
            name, value = line.split()
            out[name] = float(value)
    return out
