"""GPU parity of causal attention inside a sliding window (attn_fwd_window) against the fp64
oracle with the same window: query i sees keys i-W+1 .. i.

Small ragged cases check every row for every head dim and both 16-bit types, with windows
from a single key to more than the sequence (which is plain causal attention), dense and
packed, grouped-query heads; the tile arithmetic is exercised with windows below, at and just
past the 64- and 32-key tile sizes and the 256-query block.  Full-size cases check sampled
rows.  FP8 windows are held to the FP8 bar of tests/test_fp8_gpu.py.
"""
import numpy as np
import pytest

import seeded_inputs as si
from tests import gpu_util as gu
from tests.test_fp8_gpu import _all_rows, _full, _three_errors, check_fp8, gpu_fp8_attention

pytestmark = pytest.mark.gpu

WINDOWS = [1, 7, 32, 63, 64, 65, 100, 256, 257, 1000]


def _check_all_rows(inp, what):
    o, lse = gu.run_gpu(inp)
    o_ref, lse_ref = gu.oracle_full(inp)
    m = gu.metrics(o, o_ref, lse, lse_ref, inp.dtype)
    gu.check(m, what=what)
    return o, lse


@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("window", WINDOWS)
def test_window_dense_ragged(d, window):
    inp = si.dense_inputs(2, 300, 4, d, Hkv=2, causal=True, seed=700 + d)
    inp.window = window
    gu.say("window dense", d, window)
    _check_all_rows(inp, f"window {window} d={d}")


@pytest.mark.parametrize("window", [1, 65, 300])
def test_window_fp16(window):
    inp = si.dense_inputs(1, 520, 4, 128, causal=True, seed=701, dtype="fp16")
    inp.window = window
    gu.say("window fp16", window)
    _check_all_rows(inp, f"window {window} fp16")


def test_window_one_is_v():
    """W = 1: every row sees only itself, so O_i = V_i (P = 1, l = 1: exact) and L_i = s_ii."""
    inp = si.dense_inputs(1, 200, 4, 128, causal=True, seed=702)
    inp.window = 1
    gu.say("window one")
    o, lse = gu.run_gpu(inp)
    v = inp.widened("v").astype(np.float64)
    assert np.array_equal(o, v)


@pytest.mark.parametrize("window", [5, 64, 129, 4096])
def test_window_varlen(window):
    lengths = [1, 63, 64, 65, 200, 129, 300, 700]
    inp = si.varlen_inputs(lengths, 8, 2, 128, causal=True, seed=703)
    inp.window = window
    gu.say("window packed", window)
    _check_all_rows(inp, f"window {window} packed")


@pytest.mark.parametrize("d,window", [(128, 2048), (64, 1000), (256, 3000)])
def test_window_full_size(d, window):
    """B=2, H=16, N=8192 with a window of a few thousand keys; sampled rows."""
    inp = si.dense_inputs(2, 8192, 16, d, causal=True, seed=704)
    inp.window = window
    gu.say("window full", d, window)
    o, lse = gu.run_gpu(inp)
    heads, tokens = gu.sample_rows(inp, 1024, seed=5)
    q, k, v = gu.widened(inp)
    import oracle

    o_ref, lse_ref = oracle.attention_rows(q, k, v, heads, tokens, causal=True, alpha=inp.alpha, window=window)
    o_s, lse_s = gu.gpu_rows(inp, o, lse, heads, tokens)
    gu.check(gu.metrics(o_s, o_ref, lse_s, lse_ref, "bf16"), what=f"window {window} full d={d}")


@pytest.mark.parametrize("window", [1, 64, 100, 1000])
def test_window_fp8(window):
    inp = si.dense_inputs(2, 300, 8, 128, Hkv=2, causal=True, seed=705)
    inp.window = window
    gu.say("window fp8", window)
    o, lse, prep = gpu_fp8_attention(inp, si.hadamard_signs(128, seed=55))
    assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse))
    check_fp8(*_three_errors(inp, o, lse, prep, *_all_rows(inp)))


def test_window_fp8_packed_full():
    inp = si.CONFIGS["gqa_varlen_causal_hq32_hkv8_d128"]()
    inp.window = 2048
    gu.say("window fp8 packed full")
    _full(inp)
