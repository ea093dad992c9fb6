"""Gradients of exact attention in fp64, written from the definition.

TEST INFRASTRUCTURE ONLY (see the package docstring): nothing on the product path may import
or call this module.

Sources: the FlashAttention-3 pages -- the zenmind digest's section 4 (data path, step 5: the
backward pass recomputes P from the stored L, after a pre-processing step that forms
D = rowsum(dO * O)) and section 7.1 (backward FLOPs = 2.5 x forward: five matrix products).
The pages give no formulas for the gradients; they are the chain rule applied to the forward
definition of the digest's section 3.1, which this module writes out plainly:

  for every sequence and query head h (key/value head g = h // (Hq / Hkv)):
    S = alpha Q K^T over the visible keys, P = softmax(S) along the keys, O = P V;
  given dO (the gradient of a loss with respect to O):
    dV_g = sum over the query heads h of group g of P^T dO,
    dP   = dO V^T,
    dS   = P * (dP - D) with D_i = sum_j P_ij dP_ij  (equal to rowsum(dO * O), since O = P V),
    dQ   = alpha dS K,
    dK_g = alpha * sum over the heads h of group g of dS^T Q.

Masking (causal, sliding window, packed sequences) is that of the forward oracle: a hidden key
has P = 0, so it receives no gradient.  Every product is a float64 numpy matmul; query rows are
taken in chunks only to bound memory (the chunks are independent rows of the same formulas).
"""
from __future__ import annotations

import numpy as np

CHUNK = 1024  # query rows per step


def _visible(i: np.ndarray, n: int, causal: bool, window: int) -> np.ndarray:
    """Boolean [len(i), n]: key j visible to query i."""
    j = np.arange(n)[None, :]
    vis = np.ones((len(i), n), dtype=bool)
    if causal:
        vis &= j <= i[:, None]
    if window > 0:
        vis &= j > i[:, None] - window
    return vis


def _sequence_grads(q, k, v, do, causal, alpha, window):
    """One sequence: q, do [n, Hq, d]; k, v [n, Hkv, d] -> dq [n, Hq, d], dk, dv [n, Hkv, d]."""
    n, Hq, d = q.shape
    Hkv = k.shape[1]
    G = Hq // Hkv
    dq = np.zeros(q.shape)
    dk = np.zeros(k.shape)
    dv = np.zeros(v.shape)
    for h in range(Hq):
        g = h // G
        K, V = k[:, g, :], v[:, g, :]
        for c0 in range(0, n, CHUNK):
            rows = np.arange(c0, min(n, c0 + CHUNK))
            Q, dO = q[rows, h, :], do[rows, h, :]
            vis = _visible(rows, n, causal, window)
            S = np.where(vis, alpha * (Q @ K.T), -np.inf)
            m = np.max(S, axis=1, keepdims=True)
            E = np.where(vis, np.exp(S - m), 0.0)
            P = E / np.sum(E, axis=1, keepdims=True)
            dv[:, g, :] += P.T @ dO
            dP = dO @ V.T
            D = np.sum(P * dP, axis=1, keepdims=True)
            dS = P * (dP - D)
            dq[rows, h, :] = alpha * (dS @ K)
            dk[:, g, :] += alpha * (dS.T @ Q)
    return dq, dk, dv


def attention_backward(q, k, v, do, *, causal: bool = False, alpha: float | None = None, cu_seqlens=None,
                       window: int = 0):
    """dQ, dK, dV (float64) of O = softmax(alpha Q K^T) V for the output gradient dO.

    Dense: q, do [B, N, Hq, d], k, v [B, N, Hkv, d].  Packed: q, do [T, Hq, d], k, v [T, Hkv, d]
    with cu_seqlens [nseq + 1].  ``window`` > 0 (with causal): query i sees keys i-window+1 .. i.
    ``alpha`` defaults to 1/sqrt(d).
    """
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    d = q.shape[-1]
    alpha = 1.0 / np.sqrt(d) if alpha is None else float(alpha)
    if cu_seqlens is None:
        outs = [_sequence_grads(q[b], k[b], v[b], do[b], causal, alpha, window) for b in range(q.shape[0])]
        return tuple(np.stack([o[i] for o in outs]) for i in range(3))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    dq, dk, dv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(len(cu) - 1):
        sl = slice(cu[b], cu[b + 1])
        if cu[b + 1] > cu[b]:
            dq[sl], dk[sl], dv[sl] = _sequence_grads(q[sl], k[sl], v[sl], do[sl], causal, alpha, window)
    return dq, dk, dv


def gradient_magnitudes(q, k, v, do, *, causal: bool = False, alpha: float | None = None, cu_seqlens=None,
                        window: int = 0, row_weight=None):
    """The same products taken over absolute values (|P|^T |dO| for dV, alpha |dS| |K| for dQ,
    alpha |dS|^T |Q| for dK): the size of the sums each gradient element is, against which
    rounding errors of the factors are measured.

    With ``row_weight`` w (one value per query row and head, q's layout without d), the
    |dS| above are replaced by |dS| + P * w: the magnitudes then also bound what an error of
    up to w_i in D_i (which enters dS = P (dP - D)) does to dQ and dK."""
    q, k, v, do = (np.asarray(x, dtype=np.float64) for x in (q, k, v, do))
    d = q.shape[-1]
    alpha = 1.0 / np.sqrt(d) if alpha is None else float(alpha)

    def seq(q, k, v, do, w):
        n, Hq, _ = q.shape
        G = Hq // k.shape[1]
        mq, mk, mv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
        for h in range(Hq):
            g = h // G
            K, V = k[:, g, :], v[:, g, :]
            for c0 in range(0, n, CHUNK):
                rows = np.arange(c0, min(n, c0 + CHUNK))
                Q, dO = q[rows, h, :], do[rows, h, :]
                vis = _visible(rows, n, causal, window)
                S = np.where(vis, alpha * (Q @ K.T), -np.inf)
                E = np.where(vis, np.exp(S - np.max(S, axis=1, keepdims=True)), 0.0)
                P = E / np.sum(E, axis=1, keepdims=True)
                dP = dO @ V.T
                dS = np.abs(P * (dP - np.sum(P * dP, axis=1, keepdims=True)))
                if w is not None:
                    dS = dS + P * w[rows, h][:, None]
                mv[:, g, :] += P.T @ np.abs(dO)
                mq[rows, h, :] = alpha * (dS @ np.abs(K))
                mk[:, g, :] += alpha * (dS.T @ np.abs(Q))
        return mq, mk, mv

    w = None if row_weight is None else np.asarray(row_weight, dtype=np.float64)
    if cu_seqlens is None:
        outs = [seq(q[b], k[b], v[b], do[b], None if w is None else w[b]) for b in range(q.shape[0])]
        return tuple(np.stack([o[i] for o in outs]) for i in range(3))
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    mq, mk, mv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(len(cu) - 1):
        sl = slice(cu[b], cu[b + 1])
        if cu[b + 1] > cu[b]:
            mq[sl], mk[sl], mv[sl] = seq(q[sl], k[sl], v[sl], do[sl], None if w is None else w[sl])
    return mq, mk, mv
