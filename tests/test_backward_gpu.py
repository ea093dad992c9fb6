"""GPU parity of attn_bwd against the fp64 backward oracle (oracle/backward.py).

The GPU forward pass produces O and L, attn_bwd the gradients; the oracle differentiates the
definition directly (it never sees the GPU's O or L).  Each of dQ, dK, dV is compared element
by element with a bound built from what the kernels round (the reading is recorded with the
design notes):

  * P and dS enter their products as 16-bit values (relative error <= 2^-p, p = 8 significant
    bits for bf16, 11 for fp16), so a gradient element moves by at most 2^-p times the sum of
    the absolute values of its terms -- the oracle's gradient_magnitudes;
  * D = rowsum(dO * O) is formed from the 16-bit O, whose rounding moves D_i by at most
    w_i = 2^-p sum_c |dO_ic O_ic|; through dS = P (dP - D) that adds P_ij w_i to each |dS_ij|
    (the oracle's magnitudes with row_weight = w);
  * the result is rounded to the 16-bit output format (half an ulp).
The bound is twice the first-order sum, 2 * 2^-p * magnitude, plus half an ulp and a small
absolute floor for fp32 accumulation, per element; relative RMSE is reported too.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from oracle import backward as ob
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

SIG_BITS = {"bf16": 8, "fp16": 11}


def run_gpu_bwd(inp, do_bits):
    import exact_attention_76_amd as ea

    q, k, v, cu = gu.to_device(inp)
    do = torch.from_numpy(do_bits.view(np.int16)).view(gu.torch_dtype(inp.dtype)).cuda()
    kw = dict(causal=inp.causal, alpha=inp.alpha, cu_seqlens=cu, max_seqlen=inp.N if cu is not None else None,
              window=inp.window or None)
    o, lse = ea.attention(q, k, v, **kw)
    dq, dk, dv = ea.attention_backward(q, k, v, o, lse, do, **kw)
    torch.cuda.synchronize()
    return tuple(t.double().cpu().numpy() for t in (dq, dk, dv))


def check_grads(inp, do_bits, got, what, heads=None):
    """Compare (dq, dk, dv) with the oracle; ``heads``: restrict to these KV heads (their query
    heads' dq) to keep the oracle's work small at full size."""
    q, k, v = gu.widened(inp)
    do = oracle.widen(do_bits, inp.dtype)
    dense = inp.cu_seqlens is None
    G = inp.Hq // inp.Hkv
    if heads is not None:
        qh = np.concatenate([np.arange(g * G, (g + 1) * G) for g in heads])
        sel_q = (slice(None), slice(None), qh) if dense else (slice(None), qh)
        sel_k = (slice(None), slice(None), np.asarray(heads)) if dense else (slice(None), np.asarray(heads))
        q, do, k, v = q[sel_q], do[sel_q], k[sel_k], v[sel_k]
        got = (got[0][sel_q], got[1][sel_k], got[2][sel_k])
    kw = dict(causal=inp.causal, alpha=inp.alpha, cu_seqlens=inp.cu_seqlens, window=inp.window)
    ref = ob.attention_backward(q, k, v, do, **kw)
    u = 2.0 ** -SIG_BITS[inp.dtype]
    o_ref, _ = oracle.attention(q, k, v, **kw)
    w = np.sum(np.abs(do) * np.abs(o_ref), axis=-1)  # D's rounding error, in units of u
    mag = ob.gradient_magnitudes(q, k, v, do, **kw, row_weight=w)
    for name, g, r, m in zip(("dq", "dk", "dv"), got, ref, mag):
        bound = 2.0 * u * m + gu.half_ulp(r, inp.dtype) + 1e-5
        err = np.abs(g - r)
        rel_max = float(np.max(err) / max(np.max(np.abs(r)), 1e-30))
        rmse = float(np.sqrt(np.mean(err ** 2)) / max(np.sqrt(np.mean(r ** 2)), 1e-30))
        worst = float(np.max(err / bound))
        gu.say(f"{what} {name}: max err / max|ref| {rel_max:.2e}, relative RMSE {rmse:.2e}, worst err/bound {worst:.3f}")
        assert np.all(np.isfinite(g)), f"{what} {name}: non-finite"
        assert worst <= 1.0, f"{what} {name}: error exceeds its bound ({worst:.3f} of it)"


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("causal", [False, True])
def test_bwd_dense_ragged_gqa(d, causal):
    inp = si.dense_inputs(2, 300, 4, d, Hkv=2, causal=causal, seed=800 + d)
    do = si.output_gradient(inp, 801)
    gu.say("bwd dense", d, causal)
    check_grads(inp, do, run_gpu_bwd(inp, do), f"bwd d={d} causal={causal}")


def test_bwd_fp16():
    inp = si.dense_inputs(1, 200, 2, 128, causal=True, seed=802, dtype="fp16")
    do = si.output_gradient(inp, 803)
    gu.say("bwd fp16")
    check_grads(inp, do, run_gpu_bwd(inp, do), "bwd fp16")


@pytest.mark.parametrize("causal", [True, False])
def test_bwd_varlen(causal):
    """Packed sequences of 0 .. 300 tokens (an empty one included), GQA 8:2."""
    inp = si.varlen_inputs([1, 63, 0, 64, 65, 200, 129, 300], 8, 2, 128, causal=causal, seed=804)
    do = si.output_gradient(inp, 805)
    gu.say("bwd packed", causal)
    check_grads(inp, do, run_gpu_bwd(inp, do), f"bwd packed causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("B,N", [(300, 1), (97, 3), (33, 65)])
def test_bwd_tiny_sequences(B, N, d, causal):
    """Large batches of sequences shorter than one tile (or one key past it)."""
    inp = si.dense_inputs(B, N, 4, d, Hkv=2, causal=causal, seed=970 + B + N + d + causal)
    do = si.output_gradient(inp, 7)
    check_grads(inp, do, run_gpu_bwd(inp, do), f"bwd tiny sequences B={B} N={N} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,d", [(5, 5, 64), (7, 1, 128), (14, 7, 64), (3, 3, 128)])
def test_bwd_odd_head_counts(Hq, Hkv, d, causal):
    """Head counts that do not split evenly over the eight XCDs; dense and packed."""
    inp = si.dense_inputs(2, 217, Hq, d, Hkv=Hkv, causal=causal, seed=950 + Hq + Hkv + d)
    do = si.output_gradient(inp, 5)
    check_grads(inp, do, run_gpu_bwd(inp, do), f"bwd odd heads Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    inp = si.varlen_inputs([217, 0, 64, 300], Hq, Hkv, d, causal=causal, seed=960 + Hq + Hkv + d)
    do = si.output_gradient(inp, 6)
    check_grads(inp, do, run_gpu_bwd(inp, do), f"bwd odd heads packed Hq={Hq} Hkv={Hkv} d={d} causal={causal}")


@pytest.mark.parametrize("d", [64, 128])
def test_bwd_full_size(d):
    """B=1, N=4096, 16 heads, causal; the oracle checks two heads."""
    inp = si.dense_inputs(1, 4096, 16, d, causal=True, seed=806)
    do = si.output_gradient(inp, 807)
    gu.say("bwd full", d)
    check_grads(inp, do, run_gpu_bwd(inp, do), f"bwd full d={d}", heads=[0, 11])


def test_bwd_full_gqa_packed():
    """The packed GQA workload's shape (8 sequences, Hq=32, Hkv=8, causal); the oracle checks one
    key/value group."""
    inp = si.CONFIGS["gqa_varlen_causal_hq32_hkv8_d128"]()
    do = si.output_gradient(inp, 808)
    gu.say("bwd full packed GQA")
    check_grads(inp, do, run_gpu_bwd(inp, do), "bwd full packed GQA", heads=[5])


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("window", [1, 33, 100, 300, 1000])
def test_bwd_window(d, window):
    """Sliding windows below, at and past the tile sizes (64 keys, 32 or 64 queries, 128 and 256
    rows per workgroup) and past the sequence (plain causal)."""
    inp = si.dense_inputs(2, 700, 4, d, Hkv=2, causal=True, seed=809 + d)
    inp.window = window
    do = si.output_gradient(inp, 810)
    gu.say("bwd window", d, window)
    check_grads(inp, do, run_gpu_bwd(inp, do), f"bwd window {window} d={d}")


def test_bwd_window_packed():
    inp = si.varlen_inputs([1, 63, 0, 300, 129, 520], 8, 2, 128, causal=True, seed=811)
    inp.window = 77
    do = si.output_gradient(inp, 812)
    gu.say("bwd window packed")
    check_grads(inp, do, run_gpu_bwd(inp, do), "bwd window packed")
