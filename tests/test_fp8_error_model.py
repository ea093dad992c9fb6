"""CPU pins of the FP8 kernel's error model (tests/fp8_error_model.py), which sets the bound the
GPU tests hold the kernel's own O error to.

The model's prediction (per-weight rounding variance step^2 / 12 of e4m3, none at the row
maximum, plus the bf16 rounding of O) must agree with the same roundings carried out exactly
(the oracle's e4m3 and bf16 rounding of each weight and output) on the small FP8 cases: within
10%, so that a wrong step (a missing factor 2 in the grid, a variance of step^2 / 3), a dropped
term, or charging the exact row maximum would each fall outside.  The per-row product bound of
the LSE budget is checked against a brute-force loop."""
import numpy as np
import pytest

import oracle
from oracle import fp8 as ofp8
from tests import fp8_cases
from tests import fp8_error_model as em


def _dequantised(name):
    inp, signs, heads, tokens, per_tensor = fp8_cases.case(name)
    q, k, v = (oracle.bf16_to_f64(getattr(inp, n)) for n in "qkv")
    if inp.cu_seqlens is None:
        q8, k8, v8, qs, ks, vs = ofp8.fp8_prepare(q, k, v, signs, per_tensor=per_tensor)
        qd, kd, vd = ofp8.dequantize(q8, qs), ofp8.dequantize(k8, ks), ofp8.dequantize(v8, vs)
        T = inp.B * inp.N
        qd, kd, vd = (t.reshape(T, *t.shape[2:]) for t in (qd, kd, vd))
        cu = np.arange(inp.B + 1, dtype=np.int64) * inp.N
    else:
        q8, k8, v8, qs, ks, vs = ofp8.fp8_prepare_varlen(q, k, v, inp.cu_seqlens, inp.N, signs, per_tensor=per_tensor)
        qd, kd, vd = (ofp8.dequantize_varlen(c, sc, inp.cu_seqlens) for c, sc in ((q8, qs), (k8, ks), (v8, vs)))
        cu = inp.cu_seqlens.astype(np.int64)
    return inp, qd, kd, vd, cu, heads, tokens


SMALL = ["small_rotated", "small_unrotated", "varlen_small_causal_block", "varlen_small_noncausal_block"]


@pytest.mark.parametrize("name", SMALL)
def test_prediction_matches_emulated_roundings(name):
    inp, qd, kd, vd, cu, heads, tokens = _dequantised(name)
    kw = dict(Hq=inp.Hq, Hkv=inp.Hkv, causal=inp.causal, alpha=inp.alpha)
    pred = em.predicted_rmse(qd, kd, vd, cu, heads, tokens, **kw)
    emul = em.emulated_rmse(qd, kd, vd, cu, heads, tokens, **kw)
    assert 0.9 <= emul / pred <= 1.1, (name, pred, emul)


def test_row_maximum_carries_no_error():
    """Rows with one dominant key: the maximum weight is exactly 2^6 and the others vanish, so
    only O's bf16 rounding is left.  The model must predict that (about 2^-9 of |V|) and agree
    with the emulation; charging the maximum weight an e4m3 step would predict about 0.036 |V|."""
    rng = np.random.default_rng(3)
    R, d = 32, 128
    qd = rng.standard_normal((2 * R, 1, d))
    kd = rng.standard_normal((2 * R, 1, d)) * 0.05
    kd[R:, 0] = 4.0 * qd[:R, 0]  # key R + i dominates row i
    vd = rng.standard_normal((2 * R, 1, d))
    cu = np.array([0, 2 * R])
    kw = dict(Hq=1, Hkv=1, causal=False, alpha=0.25)
    heads, tokens = np.zeros(R, np.int64), np.arange(R)
    pred = em.predicted_rmse(qd, kd, vd, cu, heads, tokens, **kw)
    emul = em.emulated_rmse(qd, kd, vd, cu, heads, tokens, **kw)
    assert pred < 0.01 and 0.8 <= emul / pred <= 1.25, (pred, emul)


def test_max_abs_products_brute_force():
    inp, qd, kd, vd, cu, heads, tokens = _dequantised("varlen_small_causal_block")
    sel = np.arange(0, len(heads), 37)
    got = em.max_abs_products(qd, kd, cu, heads[sel], tokens[sel], Hq=inp.Hq, Hkv=inp.Hkv, causal=True)
    G = inp.Hq // inp.Hkv
    for n, r in enumerate(sel):
        h, t = int(heads[r]), int(tokens[r])
        b = int(np.searchsorted(cu, t, side="right") - 1)
        best = 0.0
        for j in range(int(cu[b]), t + 1):
            best = max(best, float(np.sum(np.abs(qd[t, h] * kd[j, h // G]))))
        assert got[n] == pytest.approx(best, rel=1e-12)
