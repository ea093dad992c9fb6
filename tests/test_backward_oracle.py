"""Pins of the backward oracle (oracle/backward.py), tied to facts outside its own formulas.

* Central finite differences of the forward oracle (the C definition of attention) on tiny
  problems, dense and packed, causal or not, with a sliding window and grouped heads: the
  directional derivative of sum(dO * O) along random perturbations of Q, K and V equals
  <dQ, E_Q> + <dK, E_K> + <dV, E_V>.
* CPU float64 torch autograd through scaled_dot_product_attention (K/V repeated for grouped
  heads, the repeats' gradients summed back).
* Invariants: the dK of one key/value head sums to zero over its keys, and its dV sums to the
  sum of dO over the visible rows' heads (each row of P sums to one); adding a constant row to
  every V leaves dQ and dK alone; dO = 0 gives zero gradients.
* Planted mistakes in copies of the oracle each fail one of these pins (test_mutation_is_caught).
"""
import importlib.util
import math
import os

import numpy as np
import pytest
import torch

import oracle
from oracle import backward as ob

SRC = os.path.join(os.path.dirname(oracle.__file__), "backward.py")


def _rand(shape, seed):
    return np.random.default_rng(seed).standard_normal(shape)


CASES = [
    # (name, dense shape or lengths, Hq, Hkv, d, causal, window)
    ("dense", (2, 6), 2, 1, 3, False, 0),
    ("dense_causal", (1, 7), 4, 2, 4, True, 0),
    ("packed_causal_window", [3, 1, 6], 2, 2, 3, True, 3),
    ("packed", [4, 5], 2, 1, 2, False, 0),
]


def _case(spec, Hq, Hkv, d, seed):
    if isinstance(spec, tuple):
        B, N = spec
        return (_rand((B, N, Hq, d), seed), _rand((B, N, Hkv, d), seed + 1), _rand((B, N, Hkv, d), seed + 2),
                _rand((B, N, Hq, d), seed + 3), None)
    cu = np.concatenate([[0], np.cumsum(spec)])
    T = int(cu[-1])
    return (_rand((T, Hq, d), seed), _rand((T, Hkv, d), seed + 1), _rand((T, Hkv, d), seed + 2),
            _rand((T, Hq, d), seed + 3), cu)


def pin_finite_differences(mod):
    for n, (name, spec, Hq, Hkv, d, causal, window) in enumerate(CASES):
        q, k, v, do, cu = _case(spec, Hq, Hkv, d, 10 * n)
        alpha = 0.7
        dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, alpha=alpha, cu_seqlens=cu, window=window)
        rng = np.random.default_rng(100 + n)
        for _ in range(3):
            eq, ek, ev = rng.standard_normal(q.shape), rng.standard_normal(k.shape), rng.standard_normal(v.shape)
            eps = 1e-5

            def loss(t):
                o, _ = oracle.attention(q + t * eq, k + t * ek, v + t * ev, causal=causal, alpha=alpha,
                                        cu_seqlens=cu, window=window)
                return math.fsum((o * do).ravel())

            fd = (loss(eps) - loss(-eps)) / (2 * eps)
            an = float(np.sum(dq * eq) + np.sum(dk * ek) + np.sum(dv * ev))
            assert abs(fd - an) <= 1e-7 * max(1.0, abs(an)), (name, fd, an)


def pin_torch_autograd(mod):
    B, N, Hq, Hkv, d = 2, 13, 4, 2, 8
    q, k, v, do = _rand((B, N, Hq, d), 1), _rand((B, N, Hkv, d), 2), _rand((B, N, Hkv, d), 3), _rand((B, N, Hq, d), 4)
    alpha = 0.3
    for causal in (False, True):
        tq = torch.from_numpy(q).permute(0, 2, 1, 3).clone().requires_grad_()
        tk = torch.from_numpy(k).permute(0, 2, 1, 3).clone().requires_grad_()
        tv = torch.from_numpy(v).permute(0, 2, 1, 3).clone().requires_grad_()
        o = torch.nn.functional.scaled_dot_product_attention(
            tq, tk.repeat_interleave(Hq // Hkv, dim=1), tv.repeat_interleave(Hq // Hkv, dim=1), is_causal=causal,
            scale=alpha)
        o.backward(torch.from_numpy(do).permute(0, 2, 1, 3))
        dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, alpha=alpha)
        for got, t in ((dq, tq), (dk, tk), (dv, tv)):
            want = t.grad.permute(0, 2, 1, 3).numpy()
            assert np.max(np.abs(got - want)) <= 1e-12 * max(1.0, np.max(np.abs(want))), causal


def pin_invariants(mod):
    B, N, Hq, Hkv, d = 1, 9, 4, 2, 5
    q, k, v, do = _rand((B, N, Hq, d), 5), _rand((B, N, Hkv, d), 6), _rand((B, N, Hkv, d), 7), _rand((B, N, Hq, d), 8)
    G = Hq // Hkv
    for causal in (False, True):
        dq, dk, dv = mod.attention_backward(q, k, v, do, causal=causal, alpha=0.5)
        assert np.max(np.abs(dk.sum(axis=1))) <= 1e-12, "dK does not sum to zero over the keys"
        want = do.reshape(B, N, Hkv, G, d).sum(axis=(1, 3))
        assert np.max(np.abs(dv.sum(axis=1) - want)) <= 1e-12, "dV does not sum to the dO rows"
        dq2, dk2, _ = mod.attention_backward(q, k, v + _rand((1, 1, Hkv, d), 9), do, causal=causal, alpha=0.5)
        assert np.max(np.abs(dq2 - dq)) <= 1e-12 and np.max(np.abs(dk2 - dk)) <= 1e-12, "V shift moved dQ or dK"
    z = mod.attention_backward(q, k, v, np.zeros_like(do), causal=True, alpha=0.5)
    assert all(np.all(x == 0) for x in z)


def pin_magnitudes_bound(mod):
    """The magnitude sums bound the gradients themselves (|sum| <= sum of |terms|)."""
    B, N, Hq, Hkv, d = 1, 11, 2, 1, 4
    q, k, v, do = _rand((B, N, Hq, d), 11), _rand((B, N, Hkv, d), 12), _rand((B, N, Hkv, d), 13), _rand((B, N, Hq, d), 14)
    g = mod.attention_backward(q, k, v, do, causal=True, alpha=0.4)
    m = mod.gradient_magnitudes(q, k, v, do, causal=True, alpha=0.4)
    for x, y in zip(g, m):
        assert np.all(np.abs(x) <= y * (1 + 1e-12) + 1e-15)


def pin_magnitudes_tight(mod):
    """The magnitude sums are exactly the gradients' sizes when every term of a sum has one sign,
    so an inflated bound (which would loosen every backward tolerance) fails here.  Two keys with
    K_1 = -K_0 make each term of dQ = alpha (dS_i0 K_0 + dS_i1 K_1) share a sign (dS_i1 = -dS_i0);
    two identical query rows (and dO rows) make the terms of dK_j = alpha sum_i dS_ij Q_i equal;
    dO >= 0 makes every term of dV = P^T dO non-negative."""
    B, N, H, d = 1, 2, 1, 4
    q1 = _rand((d,), 21)
    q = np.stack([q1, q1])[None, :, None, :]
    k0 = _rand((d,), 22)
    k = np.stack([k0, -k0])[None, :, None, :]
    v = _rand((B, N, H, d), 23)
    do1 = np.abs(_rand((d,), 24)) + 0.1
    do = np.stack([do1, do1])[None, :, None, :]
    g = mod.attention_backward(q, k, v, do, causal=False, alpha=0.4)
    m = mod.gradient_magnitudes(q, k, v, do, causal=False, alpha=0.4)
    for name, x, y in zip(("dQ", "dK", "dV"), g, m):
        assert np.max(np.abs(x)) > 1e-3, f"{name}: degenerate case"
        assert np.allclose(np.abs(x), y, rtol=1e-12, atol=1e-15), f"{name}: magnitude sum is not tight"


ALL_PINS = [pin_finite_differences, pin_torch_autograd, pin_invariants, pin_magnitudes_bound, pin_magnitudes_tight]


@pytest.mark.parametrize("pin", ALL_PINS, ids=lambda p: p.__name__)
def test_pin(pin):
    pin(ob)


MUTATIONS = {
    "no_D_term": ("dS = P * (dP - D)", "dS = P * dP"),
    "dq_without_alpha": ("dq[rows, h, :] = alpha * (dS @ K)", "dq[rows, h, :] = dS @ K"),
    "dv_from_unnormalised": ("dv[:, g, :] += P.T @ dO", "dv[:, g, :] += E.T @ dO"),
    "dk_overwrites_group": ("dk[:, g, :] += alpha * (dS.T @ Q)", "dk[:, g, :] = alpha * (dS.T @ Q)"),
    "dP_from_keys": ("            dP = dO @ V.T\n            D =", "            dP = dO @ K.T\n            D ="),
    "magnitudes_triangle": ("dS = np.abs(P * (dP - np.sum(P * dP, axis=1, keepdims=True)))",
                            "dS = P * (np.abs(dP) + np.abs(np.sum(P * dP, axis=1, keepdims=True)))"),
    "magnitudes_without_alpha": ("mq[rows, h, :] = alpha * (dS @ np.abs(K))", "mq[rows, h, :] = dS @ np.abs(K)"),
    "magnitudes_dv_unnormalised": ("mv[:, g, :] += P.T @ np.abs(dO)", "mv[:, g, :] += E.T @ np.abs(dO)"),
    "window_off_by_one": ("    if window > 0:\n        vis &= j > i[:, None] - window",
                       "    if window > 0:\n        vis &= j > i[:, None] - window - 1"),
}


@pytest.mark.parametrize("name", sorted(MUTATIONS))
def test_mutation_is_caught(name, tmp_path):
    old, new = MUTATIONS[name]
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name} not found exactly once"
    path = tmp_path / "backward_mutated.py"
    path.write_text(src.replace(old, new))
    spec = importlib.util.spec_from_file_location("backward_mutated", path)
    mod = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(mod)
    for pin in ALL_PINS:
        try:
            pin(mod)
        except AssertionError:
            return
    pytest.fail(f"no pin caught the planted mistake {name}")
