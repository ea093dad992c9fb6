"""Error model of the FP8 kernel's own arithmetic (test infrastructure).

Against exact attention on its own e4m3-dequantised inputs, the FP8 forward kernel (the
FlashAttention-3 digest's section 3.5: P is quantised to FP8 before the second product) differs
by:

* the e4m3 rounding of the weights P' = 2^6 exp(s - m) before the second product.  E4M3 keeps
  three significand bits, so a weight in the binade [2^e, 2^(e+1)) (e >= -6) lies on a grid of
  step 2^(e-3); below 2^-6 the subnormal step 2^-9 applies.  Rounding to nearest errs by at
  most half a step; taken as uniform over the step, the error's variance is step^2 / 12.  When
  the stabiliser m equals the row maximum, that weight is exactly 2^6 and carries no error.
  The row sum l is formed from the unrounded weights;
* the bf16 rounding of O (eight significand bits: step 2^(e-7) at |O| in [2^e, 2^(e+1))).

The rounding errors of different weights are independent, so the mean square error of O in row
i, column c is  sum_j var_j V_jc^2 / l_i^2  plus  step(O_ic)^2 / 12.  predicted_rmse() is the
root of that mean over the given rows and all columns.  emulated_rmse() performs the same
roundings exactly (the oracle's e4m3 and bf16 rounding) with m equal to the row maximum, which
tests/test_fp8_error_model.py uses to pin the model on the CPU.

The scores themselves carry the matrix instruction's rounding, |ds_j| <= eps * A_j with
A_j = sum_i |q_i k_ji| (eps measured by the GPU test of the instruction).  To first order a
score error moves O_c by  alpha * sum_j P_j ds_j (V_jc - O_c) / l, so score_error_bound() adds
at most  alpha * eps * sum_j P_j A_j |V_jc - O_c| / l  per element (RMS over the rows).  What
the model leaves out beyond that, and the GPU tests' 1.5x margin on the prediction covers:
between rescales the kernel's stabiliser may trail the row maximum by up to 2^2.75, which moves
the maximum weight off the e4m3 grid.
"""
from __future__ import annotations

import numpy as np

from oracle import fp8 as ofp8

P_EXP = 6          # the kernel quantises 2^6 * P
CHUNK = 256        # rows per block of the score matrix


def _groups(heads, tokens, cu):
    """Row indices grouped by (sequence, head)."""
    seq = np.searchsorted(cu, tokens, side="right") - 1
    order = np.lexsort((heads, seq))
    keys = np.stack([seq[order], heads[order]], 1)
    cut = np.flatnonzero(np.any(np.diff(keys, axis=0) != 0, axis=1)) + 1
    for part in np.split(order, cut):
        yield int(seq[part[0]]), int(heads[part[0]]), part


def _blocks(qd, kd, vd, cu, heads, tokens, *, Hq, Hkv, causal, window, alpha, products=False):
    """Per block of rows: (weights P' with m = row maximum, mask of the row maximum, V rows),
    and with ``products`` the row indices and the matrix of sum_i |q_i k_i| as well."""
    G = Hq // Hkv
    for b, h, rows in _groups(np.asarray(heads), np.asarray(tokens), np.asarray(cu, dtype=np.int64)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        K, V = kd[lo:hi, h // G], vd[lo:hi, h // G]
        for c0 in range(0, len(rows), CHUNK):
            r = rows[c0:c0 + CHUNK]
            pos = np.asarray(tokens)[r] - lo
            s = alpha * (qd[np.asarray(tokens)[r], h] @ K.T)
            j = np.arange(hi - lo)[None, :]
            hidden = np.zeros(s.shape, dtype=bool)
            if causal:
                hidden |= j > pos[:, None]
            if window:
                hidden |= j <= pos[:, None] - window
            s = np.where(hidden, -np.inf, s)
            p = 2.0 ** P_EXP * np.exp(s - s.max(axis=1, keepdims=True))
            top = np.zeros(p.shape, dtype=bool)
            top[np.arange(len(r)), np.argmax(p, axis=1)] = True
            if products:
                yield p, top, V, r, np.where(hidden, 0.0, np.abs(qd[np.asarray(tokens)[r], h]) @ np.abs(K.T))
            else:
                yield p, top, V


def _bf16_var(o):
    a = np.abs(o)
    e = np.floor(np.log2(np.where(a > 0, a, 1.0)))
    return np.where(a > 0, (2.0 ** (e - 7)) ** 2 / 12.0, 0.0)


def predicted_rmse(qd, kd, vd, cu, heads, tokens, *, Hq, Hkv, causal, alpha, window=0) -> float:
    """Model RMSE of the kernel's O against exact attention on the dequantised inputs.
    qd/kd/vd: packed [T, H, d] fp64; cu: sequence offsets; heads/tokens: the rows."""
    total, count = 0.0, 0
    for p, top, V in _blocks(qd, kd, vd, cu, heads, tokens, Hq=Hq, Hkv=Hkv, causal=causal, window=window,
                             alpha=alpha):
        e = np.floor(np.log2(np.where(p > 0, p, 1.0)))
        step = np.where(p >= 2.0 ** -6, 2.0 ** (e - 3), 2.0 ** -9)
        var = np.where(top | (p == 0), 0.0, step ** 2 / 12.0)
        l = p.sum(axis=1, keepdims=True)
        o = (p @ V) / l
        total += float(np.sum((var @ (V * V)) / l ** 2) + np.sum(_bf16_var(o)))
        count += o.size
    return float(np.sqrt(total / count))


def emulated_rmse(qd, kd, vd, cu, heads, tokens, *, Hq, Hkv, causal, alpha, window=0) -> float:
    """The same roundings carried out: P' through e4m3 (the oracle's codec), l from the
    unrounded P', O rounded to bf16, against exact O."""
    total, count = 0.0, 0
    for p, _, V in _blocks(qd, kd, vd, cu, heads, tokens, Hq=Hq, Hkv=Hkv, causal=causal, window=window,
                           alpha=alpha):
        pq = ofp8.e4m3_decode(ofp8.e4m3_encode(p))
        l = p.sum(axis=1, keepdims=True)
        exact = (p @ V) / l
        got = ofp8.bf16_round((pq @ V) / l).astype(np.float64)
        total += float(np.sum((got - exact) ** 2))
        count += exact.size
    return float(np.sqrt(total / count))


def max_abs_products(qd, kd, cu, heads, tokens, *, Hq, Hkv, causal, window=0) -> np.ndarray:
    """Per row (in the given order): the largest, over the keys the row sees, of
    sum_i |q_i k_i|, the scale of the rounding error of that score's dot product."""
    out = np.zeros(len(heads))
    G = Hq // Hkv
    tokens = np.asarray(tokens)
    for b, h, rows in _groups(np.asarray(heads), tokens, np.asarray(cu, dtype=np.int64)):
        lo, hi = int(cu[b]), int(cu[b + 1])
        K = np.abs(kd[lo:hi, h // G])
        for c0 in range(0, len(rows), CHUNK):
            r = rows[c0:c0 + CHUNK]
            pos = tokens[r] - lo
            a = np.abs(qd[tokens[r], h]) @ K.T
            j = np.arange(hi - lo)[None, :]
            hidden = np.zeros(a.shape, dtype=bool)
            if causal:
                hidden |= j > pos[:, None]
            if window:
                hidden |= j <= pos[:, None] - window
            out[r] = np.where(hidden, 0.0, a).max(axis=1)
    return out


def score_error_bound(qd, kd, vd, cu, heads, tokens, *, eps, Hq, Hkv, causal, alpha, window=0) -> float:
    """RMS over the rows and columns of the first-order bound on the O error that score errors
    |ds_j| <= eps * sum_i |q_i k_ji| cause: alpha * eps * sum_j P_j A_j |V_jc - O_c| / l."""
    total, count = 0.0, 0
    for p, _, V, _, A in _blocks(qd, kd, vd, cu, heads, tokens, Hq=Hq, Hkv=Hkv, causal=causal, window=window,
                                 alpha=alpha, products=True):
        l = p.sum(axis=1, keepdims=True)
        o = (p @ V) / l
        w = p * A / l                                          # rows x keys
        for r0 in range(0, len(p), 8):                         # rows x keys x d, eight rows at a time
            dev = np.abs(V[None, :, :] - o[r0:r0 + 8, None, :])
            b = alpha * eps * np.einsum("rk,rkd->rd", w[r0:r0 + 8], dev)
            total += float(np.sum(b * b))
            count += b.size
    return float(np.sqrt(total / count))
