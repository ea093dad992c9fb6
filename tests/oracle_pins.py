"""Pins that tie the fp64 attention oracle to facts outside itself.

Each ``pin_*`` function takes an :class:`oracle.OracleLib` and raises AssertionError when the
oracle it is handed disagrees with a closed form, an invariant, a brute-force evaluation in
50-digit arithmetic, a library routine or the blockwise recurrences of the pages' Algorithm 1.
The same functions run against the real oracle (test_oracle_pins.py) and against copies of it
with planted mistakes (test_oracle_mutations.py), so every plausible slip is shown to fail at
least one of them.

Definition being pinned (FlashAttention-3 digest, section 3.1): S = alpha Q K^T,
P = softmax(S) along keys after subtracting the row maximum, O = P V; L = m + log(l)
(section 3.2, Algorithm-1 epilogue).
"""
from __future__ import annotations

import math
import os

import mpmath
import numpy as np
import torch

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


def _close(a, b, tol, what):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, f"{what}: shape {a.shape} vs {b.shape}"
    assert np.all(np.isfinite(a)), f"{what}: non-finite values"
    err = float(np.max(np.abs(a - b))) if a.size else 0.0
    assert err <= tol, f"{what}: max error {err:.3e} > {tol:.1e}"


# --- closed forms -------------------------------------------------------------------------

def pin_causal_first_row(lib):
    """Causal row 0 sees only key 0: O_0 = V_0 exactly and L_0 = s_00."""
    B, N, Hq, Hkv, d = 2, 7, 4, 2, 8
    q, k, v = _rand((B, N, Hq, d), 1), _rand((B, N, Hkv, d), 2), _rand((B, N, Hkv, d), 3)
    alpha = 0.37
    o, lse = lib.attention(q, k, v, causal=True, alpha=alpha)
    for b in range(B):
        for h in range(Hq):
            g = h // (Hq // Hkv)
            assert np.array_equal(o[b, 0, h], v[b, 0, g]), "causal row 0 is not a copy of V_0"
            s00 = alpha * math.fsum(q[b, 0, h] * k[b, 0, g])
            assert abs(lse[b, h, 0] - s00) <= 1e-14 * max(1.0, abs(s00)), "L_0 != s_00"
    # varlen: the first token of every sequence
    cu = np.array([0, 3, 4, 9])
    T = 9
    q, k, v = _rand((T, Hq, d), 4), _rand((T, Hkv, d), 5), _rand((T, Hkv, d), 6)
    o, lse = lib.attention(q, k, v, causal=True, alpha=alpha, cu_seqlens=cu)
    for t0 in cu[:-1]:
        for h in range(Hq):
            g = h // (Hq // Hkv)
            assert np.array_equal(o[t0, h], v[t0, g])
            s00 = alpha * math.fsum(q[t0, h] * k[t0, g])
            assert abs(lse[h, t0] - s00) <= 1e-14 * max(1.0, abs(s00))


def pin_uniform_scores(lib):
    """Q = 0 makes every score 0: O_i is the mean of the visible V rows and L_i = ln |A(i)|."""
    B, N, Hq, Hkv, d = 2, 6, 4, 2, 5
    k, v = _rand((B, N, Hkv, d), 7), _rand((B, N, Hkv, d), 8)
    q = np.zeros((B, N, Hq, d))
    for causal in (False, True):
        o, lse = lib.attention(q, k, v, causal=causal, alpha=0.5)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            if causal:
                counts = np.arange(1, N + 1, dtype=np.float64)
                mean = np.cumsum(v[:, :, g, :], axis=1) / counts[None, :, None]
            else:
                counts = np.full(N, float(N))
                mean = np.repeat(v[:, :, g, :].mean(axis=1, keepdims=True), N, axis=1)
            _close(o[:, :, h, :], mean, 1e-14, f"uniform causal={causal} O")
            _close(lse[:, h, :], np.log(counts)[None, :].repeat(B, 0), 1e-14, "uniform L")
    # varlen with a length-1 sequence
    cu = np.array([0, 1, 5, 7])
    T = 7
    k, v = _rand((T, Hkv, d), 9), _rand((T, Hkv, d), 10)
    q = np.zeros((T, Hq, d))
    o, lse = lib.attention(q, k, v, causal=False, cu_seqlens=cu)
    for s in range(3):
        a, b = cu[s], cu[s + 1]
        for h in range(Hq):
            g = h // (Hq // Hkv)
            _close(o[a:b, h], np.repeat(v[a:b, g].mean(0, keepdims=True), b - a, 0), 1e-14, "varlen mean")
            _close(lse[h, a:b], np.full(b - a, math.log(b - a)), 1e-14, "varlen L")


def _one_hot_case(N, d, jstar, c):
    q = np.zeros((1, N, 1, d))
    q[0, :, 0, 0] = c
    k = np.zeros((1, N, 1, d))
    k[0, jstar, 0, 0] = 1.0
    v = _rand((1, N, 1, d), 11)
    return q, k, v


def pin_one_hot_key(lib):
    """One key aligned with every query: O_i = (e^x V_j* + sum_{j != j*} V_j) / (e^x + n - 1),
    L = ln(e^x + n - 1) with x = alpha c; for x = 800 this is a copy of V_j* and L = 800 (a
    missing max subtraction overflows there)."""
    N, d, jstar = 9, 4, 5
    alpha = 0.5
    for x in (2.0, 800.0):
        q, k, v = _one_hot_case(N, d, jstar, x / alpha)
        o, lse = lib.attention(q, k, v, causal=False, alpha=alpha)
        rest = v[0, :, 0].sum(0) - v[0, jstar, 0]
        if x < 700:
            ex = math.exp(x)
            want = (ex * v[0, jstar, 0] + rest) / (ex + N - 1)
            want_l = math.log(ex + N - 1)
        else:
            want = v[0, jstar, 0]
            want_l = x
        for i in range(N):
            _close(o[0, i, 0], want, 1e-14, f"one-hot x={x} O")
            _close(lse[0, 0, i], want_l, 1e-13, f"one-hot x={x} L")
        # causal: before j* the key is invisible, afterwards it dominates as above
        o, lse = lib.attention(q, k, v, causal=True, alpha=alpha)
        for i in range(N):
            vis = v[0, : i + 1, 0]
            if i < jstar:
                _close(o[0, i, 0], vis.mean(0), 1e-14, "one-hot causal pre")
                _close(lse[0, 0, i], math.log(i + 1), 1e-14, "one-hot causal pre L")
            elif x < 700:
                ex = math.exp(x)
                want = (ex * v[0, jstar, 0] + vis.sum(0) - v[0, jstar, 0]) / (ex + i)
                _close(o[0, i, 0], want, 1e-14, "one-hot causal post")
                _close(lse[0, 0, i], math.log(ex + i), 1e-13, "one-hot causal post L")
            else:
                _close(o[0, i, 0], v[0, jstar, 0], 1e-14, "one-hot causal post (copy)")
                _close(lse[0, 0, i], x, 1e-13, "one-hot causal post L")


def pin_golden_weights(lib):
    """Worked example from tests/golden/weighted_mean.txt (scores ln w_j give weights w_j)."""
    path = os.path.join(GOLDEN, "weighted_mean.txt")
    rows = [l.split() for l in open(path) if l.strip() and not l.startswith("#")]
    w = np.array([float(x) for x in rows[0][1:]])
    vals = np.array([[float(x) for x in r[1:]] for r in rows[1:] if r[0] == "v"])
    want_nc = [float(x) for x in next(r for r in rows if r[0] == "o_noncausal")[1:]]
    want_l_nc = float(next(r for r in rows if r[0] == "lse_noncausal")[1])
    want_c = [[float(x) for x in r[1:]] for r in rows if r[0] == "o_causal"]
    want_l_c = [float(x) for x in next(r for r in rows if r[0] == "lse_causal")[1:]]
    n = len(w)
    q = np.zeros((1, n, 1, 2))
    q[0, :, 0, 0] = 1.0
    k = np.zeros((1, n, 1, 2))
    k[0, :, 0, 0] = np.log(w)
    v = vals.reshape(1, n, 1, 2)
    o, lse = lib.attention(q, k, v, causal=False, alpha=1.0)
    for i in range(n):
        _close(o[0, i, 0], want_nc, 1e-14, "golden O non-causal")
        _close(lse[0, 0, i], want_l_nc, 1e-14, "golden L non-causal")
    o, lse = lib.attention(q, k, v, causal=True, alpha=1.0)
    _close(o[0, :, 0], np.array(want_c), 1e-14, "golden O causal")
    _close(lse[0, 0], np.array(want_l_c), 1e-14, "golden L causal")


# --- brute force and library cross-checks ------------------------------------------------

def _mp_attention(q, k, v, cu, causal, alpha, Hq, Hkv, window=0):
    """50-digit softmax attention, row by row, straight from the definition (window > 0: keys
    j > t - window only)."""
    mpmath.mp.dps = 50
    T, _, d = q.shape
    o = np.zeros((T, Hq, d))
    lse = np.zeros((Hq, T))
    a = mpmath.mpf(alpha)
    for s in range(len(cu) - 1):
        st, en = int(cu[s]), int(cu[s + 1])
        for t in range(st, en):
            for h in range(Hq):
                g = h // (Hq // Hkv)
                keys = range(st, t + 1) if causal else range(st, en)
                if window > 0:
                    keys = [j for j in keys if j > t - window]
                sc = [a * mpmath.fsum(mpmath.mpf(q[t, h, c]) * mpmath.mpf(k[j, g, c]) for c in range(d))
                      for j in keys]
                e = [mpmath.exp(x) for x in sc]
                z = mpmath.fsum(e)
                for c in range(d):
                    o[t, h, c] = float(mpmath.fsum(e[n] * mpmath.mpf(v[j, g, c])
                                                   for n, j in enumerate(keys)) / z)
                lse[h, t] = float(mpmath.log(z))
    return o, lse


def pin_bruteforce_mpmath(lib):
    """Tiny problems (N <= 16, d <= 8) against 50-digit arithmetic."""
    cases = [(np.array([0, 5]), 2, 1, 3), (np.array([0, 2, 7, 16]), 4, 2, 8)]
    for n, (cu, Hq, Hkv, d) in enumerate(cases):
        T = int(cu[-1])
        q, k, v = _rand((T, Hq, d), 20 + n), _rand((T, Hkv, d), 30 + n), _rand((T, Hkv, d), 40 + n)
        alpha = 1.0 / math.sqrt(d)
        for causal in (False, True):
            o, lse = lib.attention(q, k, v, causal=causal, alpha=alpha, cu_seqlens=cu)
            o_mp, lse_mp = _mp_attention(q, k, v, cu, causal, alpha, Hq, Hkv)
            _close(o, o_mp, 1e-14, f"mpmath O case {n} causal={causal}")
            _close(lse, lse_mp, 1e-14, f"mpmath L case {n} causal={causal}")


def pin_torch_sdpa(lib):
    """CPU float64 torch scaled_dot_product_attention (K/V repeated per head group); L from
    torch.logsumexp over the masked scaled scores."""
    B, N, Hq, Hkv, d = 2, 33, 6, 2, 16
    q, k, v = _rand((B, N, Hq, d), 50), _rand((B, N, Hkv, d), 51), _rand((B, N, Hkv, d), 52)
    alpha = 0.21
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    for causal in (False, True):
        ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, is_causal=causal, scale=alpha)
        s = alpha * (tq @ tk.transpose(-1, -2))
        if causal:
            s = s.masked_fill(torch.ones(N, N, dtype=torch.bool).triu(1), float("-inf"))
        ref_l = torch.logsumexp(s, dim=-1)
        o, lse = lib.attention(q, k, v, causal=causal, alpha=alpha)
        _close(o, ref.permute(0, 2, 1, 3).numpy(), 1e-13, f"sdpa O causal={causal}")
        _close(lse, ref_l.numpy(), 1e-13, f"sdpa L causal={causal}")


# --- invariants ---------------------------------------------------------------------------

def pin_invariants(lib):
    B, N, Hq, Hkv, d = 1, 12, 4, 2, 6
    q, k, v = _rand((B, N, Hq, d), 60), _rand((B, N, Hkv, d), 61), _rand((B, N, Hkv, d), 62)
    o, lse = lib.attention(q, k, v, causal=False)
    # joint permutation of key/value rows (non-causal)
    perm = np.random.default_rng(63).permutation(N)
    o2, lse2 = lib.attention(q, k[:, perm], v[:, perm], causal=False)
    _close(o2, o, 1e-13, "key permutation O")
    _close(lse2, lse, 1e-13, "key permutation L")
    # shifting every key by u leaves O alone and shifts L_i by alpha <q_i, u>
    alpha = 1.0 / math.sqrt(d)
    u = 1e3 * _rand((d,), 64)
    for causal in (False, True):
        o_c, lse_c = lib.attention(q, k, v, causal=causal)
        o3, lse3 = lib.attention(q, k + u, v, causal=causal)
        shift = alpha * np.einsum("bnhd,d->bhn", q, u)
        _close(o3, o_c, 1e-9, f"key shift O causal={causal}")
        _close(lse3 - shift, lse_c, 1e-9, f"key shift L causal={causal}")
    # affine in V
    a, bvec = -2.5, _rand((d,), 65)
    o4, lse4 = lib.attention(q, k, a * v + bvec, causal=True)
    o_c, lse_c = lib.attention(q, k, v, causal=True)
    _close(o4, a * o_c + bvec, 1e-13, "affine V")
    _close(lse4, lse_c, 0.0, "affine V leaves L")
    # GQA equals MHA with K/V replicated per group
    kr = np.repeat(k, Hq // Hkv, axis=2)
    vr = np.repeat(v, Hq // Hkv, axis=2)
    for causal in (False, True):
        og, lg = lib.attention(q, k, v, causal=causal)
        om, lm = lib.attention(q, kr, vr, causal=causal)
        _close(og, om, 0.0, "GQA vs replicated MHA O")
        _close(lg, lm, 0.0, "GQA vs replicated MHA L")
    # varlen equals independent runs per sequence, and dense equals varlen with equal lengths
    cu = np.array([0, 4, 5, 12])
    qp, kp, vp = q[0], k[0], v[0]
    ov, lv = lib.attention(qp, kp, vp, causal=True, cu_seqlens=cu)
    for s in range(3):
        a0, a1 = cu[s], cu[s + 1]
        os_, ls_ = lib.attention(q[:, a0:a1], k[:, a0:a1], v[:, a0:a1], causal=True)
        _close(ov[a0:a1], os_[0], 0.0, "varlen vs per-sequence O")
        _close(lv[:, a0:a1], ls_[0], 0.0, "varlen vs per-sequence L")
    q2, k2, v2 = _rand((3, 5, Hq, d), 66), _rand((3, 5, Hkv, d), 67), _rand((3, 5, Hkv, d), 68)
    od, ld = lib.attention(q2, k2, v2, causal=True)
    ov, lv = lib.attention(q2.reshape(15, Hq, d), k2.reshape(15, Hkv, d), v2.reshape(15, Hkv, d),
                           causal=True, cu_seqlens=np.array([0, 5, 10, 15]))
    _close(od.reshape(15, Hq, d), ov, 0.0, "dense vs varlen O")
    _close(ld.transpose(1, 0, 2).reshape(Hq, 15), lv, 0.0, "dense vs varlen L")


def pin_empty_sequences(lib):
    """Zero-length sequences anywhere in a pack (first, middle, last, and two in a row) own no
    tokens: every token still belongs to the sequence that holds it, so the packed result equals
    independent runs of the non-empty sequences, through both entry points."""
    Hq, Hkv, d = 4, 2, 6
    lengths = [0, 4, 0, 0, 1, 7, 0]
    cu = np.concatenate([[0], np.cumsum(lengths)])
    T = int(cu[-1])
    q, k, v = _rand((T, Hq, d), 90), _rand((T, Hkv, d), 91), _rand((T, Hkv, d), 92)
    for causal in (False, True):
        o, lse = lib.attention(q, k, v, causal=causal, cu_seqlens=cu)
        for s in range(len(lengths)):
            a0, a1 = cu[s], cu[s + 1]
            if a1 == a0:
                continue
            os_, ls_ = lib.attention(q[None, a0:a1], k[None, a0:a1], v[None, a0:a1], causal=causal)
            _close(o[a0:a1], os_[0], 0.0, "packed with empty sequences vs per-sequence O")
            _close(lse[:, a0:a1], ls_[0], 0.0, "packed with empty sequences vs per-sequence L")
        hs, ts = np.repeat(np.arange(Hq), T), np.tile(np.arange(T), Hq)
        orow, lrow = lib.attention_rows(q, k, v, hs, ts, causal=causal, cu_seqlens=cu)
        _close(orow, o[ts, hs], 0.0, "rows with empty sequences O")
        _close(lrow, lse[hs, ts], 0.0, "rows with empty sequences L")


def pin_rows_match_full(lib):
    """The sampled-row entry point returns exactly the rows of the full computation."""
    cu = np.array([0, 9, 30, 31])
    T, Hq, Hkv, d = 31, 4, 1, 8
    q, k, v = _rand((T, Hq, d), 70), _rand((T, Hkv, d), 71), _rand((T, Hkv, d), 72)
    o, lse = lib.attention(q, k, v, causal=True, cu_seqlens=cu)
    rng = np.random.default_rng(73)
    hs, ts = rng.integers(0, Hq, 40), rng.integers(0, T, 40)
    orow, lrow = lib.attention_rows(q, k, v, hs, ts, causal=True, cu_seqlens=cu)
    _close(orow, o[ts, hs], 0.0, "rows O")
    _close(lrow, lse[hs, ts], 0.0, "rows L")


# --- Algorithm 1 (tiled, online softmax) equals the definition -----------------------------

def blockwise_algorithm1(q, k, v, causal, alpha, Br, Bc):
    """Test-only numpy restatement of the pages' Algorithm 1 for one head: per query block,
    running max m, running sum l and an O accumulator rescaled by exp(m_old - m_new) over
    key blocks; epilogue O / l and L = m + log l."""
    N, d = q.shape
    o = np.zeros((N, d))
    L = np.zeros(N)
    for i0 in range(0, N, Br):
        qi = q[i0:i0 + Br]
        rows = np.arange(i0, i0 + len(qi))
        m = np.full(len(qi), -np.inf)
        l = np.zeros(len(qi))
        acc = np.zeros((len(qi), d))
        for j0 in range(0, N, Bc):
            kj, vj = k[j0:j0 + Bc], v[j0:j0 + Bc]
            s = alpha * qi @ kj.T
            if causal:
                cols = np.arange(j0, j0 + len(kj))
                s = np.where(cols[None, :] <= rows[:, None], s, -np.inf)
            m_new = np.maximum(m, s.max(axis=1))
            base = np.where(np.isfinite(m_new), m_new, 0.0)
            p = np.exp(s - base[:, None])
            corr = np.exp(np.where(np.isfinite(m), m, -np.inf) - base)
            l = corr * l + p.sum(axis=1)
            acc = corr[:, None] * acc + p @ vj
            m = m_new
        o[i0:i0 + Br] = acc / l[:, None]
        L[i0:i0 + Br] = m + np.log(l)
    return o, L


def pin_algorithm1(lib):
    N, d = 45, 8
    q, k, v = _rand((1, N, 1, d), 80), _rand((1, N, 1, d), 81), _rand((1, N, 1, d), 82)
    alpha = 1.0 / math.sqrt(d)
    for causal in (False, True):
        o, lse = lib.attention(q, k, v, causal=causal, alpha=alpha)
        for Br, Bc in ((16, 16), (8, 32), (45, 7)):
            ob, lb = blockwise_algorithm1(q[0, :, 0], k[0, :, 0], v[0, :, 0], causal, alpha, Br, Bc)
            _close(ob, o[0, :, 0], 1e-13, f"Alg.1 O Br={Br} Bc={Bc} causal={causal}")
            _close(lb, lse[0, 0], 1e-13, f"Alg.1 L Br={Br} Bc={Bc} causal={causal}")


# --- sliding window -------------------------------------------------------------------------

def pin_sliding_window(lib):
    """Causal attention inside a window of W keys (query i sees keys i-W+1 .. i):
    * Q = 0: O_i is the mean of the last min(W, i+1) V rows and L_i = ln min(W, i+1);
    * W = 1: O_i = V_i exactly and L_i = s_ii;
    * W >= N is plain causal attention, bit for bit;
    * 50-digit brute force on packed sequences with W = 3;
    * CPU float64 torch scaled_dot_product_attention with the band mask as attn_mask."""
    B, N, Hq, Hkv, d = 2, 9, 4, 2, 5
    k, v = _rand((B, N, Hkv, d), 70), _rand((B, N, Hkv, d), 71)
    q0 = np.zeros((B, N, Hq, d))
    for W in (1, 3, 4):
        o, lse = lib.attention(q0, k, v, causal=True, alpha=0.5, window=W)
        counts = np.minimum(np.arange(1, N + 1), W).astype(np.float64)
        for h in range(Hq):
            g = h // (Hq // Hkv)
            mean = np.stack([v[:, max(0, i - W + 1):i + 1, g].mean(axis=1) for i in range(N)], axis=1)
            _close(o[:, :, h], mean, 1e-14, f"window {W} uniform O")
            _close(lse[:, h], np.log(counts)[None].repeat(B, 0), 1e-14, f"window {W} uniform L")
    q = _rand((B, N, Hq, d), 72)
    alpha = 0.4
    o, lse = lib.attention(q, k, v, causal=True, alpha=alpha, window=1)
    for h in range(Hq):
        g = h // (Hq // Hkv)
        assert np.array_equal(o[:, :, h], v[:, :, g]), "window 1 is not a copy of V_i"
        s_ii = alpha * np.einsum("bnd,bnd->bn", q[:, :, h], k[:, :, g])
        _close(lse[:, h], s_ii, 1e-14, "window 1 L")
    o_c, lse_c = lib.attention(q, k, v, causal=True, alpha=alpha)
    for W in (N, N + 5):
        o_w, lse_w = lib.attention(q, k, v, causal=True, alpha=alpha, window=W)
        assert np.array_equal(o_w, o_c) and np.array_equal(lse_w, lse_c), f"window {W} >= N is not causal"
    cu = np.array([0, 2, 7, 13])
    T = 13
    qv, kv, vv = _rand((T, 2, 4), 73), _rand((T, 1, 4), 74), _rand((T, 1, 4), 75)
    o, lse = lib.attention(qv, kv, vv, causal=True, alpha=0.5, cu_seqlens=cu, window=3)
    o_mp, lse_mp = _mp_attention(qv, kv, vv, cu, True, 0.5, 2, 1, window=3)
    _close(o, o_mp, 1e-14, "window mpmath O")
    _close(lse, lse_mp, 1e-14, "window mpmath L")
    N2, W = 40, 7
    q, k, v = _rand((1, N2, Hq, 8), 76), _rand((1, N2, Hkv, 8), 77), _rand((1, N2, Hkv, 8), 78)
    tq = torch.from_numpy(q).permute(0, 2, 1, 3)
    tk = torch.from_numpy(k).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    tv = torch.from_numpy(v).permute(0, 2, 1, 3).repeat_interleave(Hq // Hkv, dim=1)
    i, j = np.arange(N2)[:, None], np.arange(N2)[None, :]
    band = torch.from_numpy((j <= i) & (j > i - W))
    ref = torch.nn.functional.scaled_dot_product_attention(tq, tk, tv, attn_mask=band, scale=0.3)
    ref_l = torch.logsumexp((0.3 * (tq @ tk.transpose(-1, -2))).masked_fill(~band, float("-inf")), dim=-1)
    o, lse = lib.attention(q, k, v, causal=True, alpha=0.3, window=W)
    _close(o, ref.permute(0, 2, 1, 3).numpy(), 1e-13, "window sdpa O")
    _close(lse, ref_l.numpy(), 1e-13, "window sdpa L")


ALL_PINS = [pin_causal_first_row, pin_uniform_scores, pin_one_hot_key, pin_golden_weights,
            pin_bruteforce_mpmath, pin_torch_sdpa, pin_invariants, pin_empty_sequences, pin_rows_match_full,
            pin_algorithm1, pin_sliding_window]
