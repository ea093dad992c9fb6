"""GPU parity on seeded random problem shapes: each case draws batch or packed sequence lengths,
head counts (any grouping), head dim, mask (none, causal, causal sliding window) and 16-bit
dtype, or the FP8 path with its pre-pass (block scales, or for every other FP8 draw one scale
per tensor), and compares every element of O and L with the fp64 oracle on the same inputs.  The hand-picked cases of the other test files cover each code path
on purpose; these cover combinations of them.  Sizes stay small (at most about 1000 tokens per
sequence) so the oracle runs every row in seconds.

Bars: the 16-bit ones of tests/test_parity_gpu.py; for FP8 the 3e-2 bar against fp64 on the
unquantised inputs (N(0,1) inputs, no outliers: the quantisation floor is far below it) and the
kernel's own-error bounds of tests/test_fp8_gpu.py.  The backward cases (16-bit, d = 64 or 128)
are held to the per-element bounds of tests/test_backward_gpu.py."""
import numpy as np
import pytest

import seeded_inputs as si
from tests import gpu_util as gu
from tests.test_backward_gpu import check_grads, run_gpu_bwd
from tests.test_fp8_gpu import _all_rows, _three_errors, check_fp8, gpu_fp8_attention

N_CASES = 48
N_BWD = 16


def _draw(case: int):
    """One random problem (seeded by the case index)."""
    rng = np.random.default_rng(9000 + case)
    fp8 = case % 4 == 3
    d = 128 if fp8 else int(rng.choice([64, 128, 256]))
    Hkv = int(rng.choice([1, 2, 4, 8]))
    Hq = Hkv * int(rng.choice([1, 2, 3, 4]))
    mode = rng.choice(["none", "causal", "window"])
    dtype = "bf16" if fp8 else str(rng.choice(["bf16", "fp16"]))
    seed = int(rng.integers(1 << 30))
    if rng.random() < 0.5:
        B = int(rng.integers(1, 4))
        N = int(rng.integers(1, 1000))
        inp = si.dense_inputs(B, N, Hq, d, Hkv=Hkv, causal=mode != "none", seed=seed, dtype=dtype)
    else:
        lengths = [int(x) for x in rng.integers(1, 800, int(rng.integers(1, 6)))]
        if rng.random() < 1 / 3:  # an empty sequence somewhere in the pack
            lengths.insert(int(rng.integers(0, len(lengths) + 1)), 0)
        inp = si.varlen_inputs(lengths, Hq, Hkv, d, causal=mode != "none", seed=seed, dtype=dtype)
    if mode == "window":
        inp.window = int(rng.integers(1, max(2, inp.N + 50)))
    return inp, fp8


def _per_tensor(case: int) -> bool:
    """FP8 draws alternate between block and per-tensor scales (by case index, so the seeded
    draws themselves do not change)."""
    return case % 8 == 7


def _describe(inp, fp8):
    cu = None if inp.cu_seqlens is None else np.diff(inp.cu_seqlens).tolist()
    return (f"{'fp8' if fp8 else inp.dtype} B={inp.B} N={inp.N} Hq={inp.Hq} Hkv={inp.Hkv} d={inp.d} "
            f"causal={inp.causal} window={inp.window} lengths={cu}")


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_CASES))
def test_random_shape(case):
    inp, fp8 = _draw(case)
    what = _describe(inp, fp8)
    gu.say("random shape", case, what, "per-tensor scales" if fp8 and _per_tensor(case) else "")
    if fp8:
        o, lse, prep = gpu_fp8_attention(inp, si.hadamard_signs(128, seed=55), per_tensor=_per_tensor(case))
        assert np.all(np.isfinite(o)) and np.all(np.isfinite(lse)), "rows left unwritten"
        check_fp8(*_three_errors(inp, o, lse, prep, *_all_rows(inp)))
        return
    o_gpu, lse_gpu = gu.run_gpu(inp)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), "rows left unwritten"
    o_ref, lse_ref = gu.oracle_full(inp)
    gu.check(gu.metrics(o_gpu, o_ref, lse_gpu, lse_ref, inp.dtype), what=what)


def _draw_bwd(case: int):
    """One random backward problem: 16-bit, d = 64 or 128, up to about 600 tokens per sequence."""
    rng = np.random.default_rng(9500 + case)
    d = int(rng.choice([64, 128]))
    Hkv = int(rng.choice([1, 2, 4]))
    Hq = Hkv * int(rng.choice([1, 2, 4]))
    mode = rng.choice(["none", "causal", "window"])
    dtype = str(rng.choice(["bf16", "fp16"]))
    seed = int(rng.integers(1 << 30))
    if rng.random() < 0.5:
        inp = si.dense_inputs(int(rng.integers(1, 3)), int(rng.integers(1, 600)), Hq, d, Hkv=Hkv,
                              causal=mode != "none", seed=seed, dtype=dtype)
    else:
        lengths = [int(x) for x in rng.integers(0, 500, int(rng.integers(1, 5)))]
        if sum(lengths) == 0:
            lengths[0] = 1
        inp = si.varlen_inputs(lengths, Hq, Hkv, d, causal=mode != "none", seed=seed, dtype=dtype)
    if mode == "window":
        inp.window = int(rng.integers(1, max(2, inp.N + 50)))
    return inp, seed


@pytest.mark.gpu
@pytest.mark.parametrize("case", range(N_BWD))
def test_random_shape_backward(case):
    inp, seed = _draw_bwd(case)
    what = "bwd " + _describe(inp, False)
    gu.say("random backward shape", case, what)
    do = si.output_gradient(inp, seed + 1)
    check_grads(inp, do, run_gpu_bwd(inp, do), what)


def test_draws_cover_the_modes():
    """The seeded draws include every mode, head dim, dtype and both layouts (CPU check of the
    generator, so a change of seeds cannot silently drop a combination)."""
    seen = set()
    for c in range(N_CASES):
        inp, fp8 = _draw(c)
        seen.add(("fp8" if fp8 else inp.dtype, inp.d, "window" if inp.window else ("causal" if inp.causal else "none"),
                  inp.cu_seqlens is not None))
    assert {k[0] for k in seen} == {"bf16", "fp16", "fp8"}
    fp8_cases = [c for c in range(N_CASES) if _draw(c)[1]]
    assert {_per_tensor(c) for c in fp8_cases} == {False, True}, "FP8 draws must use both scalings"
    assert {k[1] for k in seen} == {64, 128, 256}
    assert {k[2] for k in seen} == {"none", "causal", "window"}
    assert {k[3] for k in seen} == {False, True}
    assert any(inp.cu_seqlens is not None and np.any(np.diff(inp.cu_seqlens) == 0)
               for inp, _ in map(_draw, range(N_CASES))), "no packed draw with an empty sequence"
    seen = set()
    for c in range(N_BWD):
        inp, _ = _draw_bwd(c)
        seen.add((inp.dtype, inp.d, "window" if inp.window else ("causal" if inp.causal else "none"),
                  inp.cu_seqlens is not None))
    assert {k[0] for k in seen} == {"bf16", "fp16"} and {k[1] for k in seen} == {64, 128}
    assert {k[2] for k in seen} == {"none", "causal", "window"} and {k[3] for k in seen} == {False, True}
