"""Pins of the FP8 pre-pass oracle (oracle/fp8.py).

* e4m3: the OCP 8-bit floating point specification (E4M3: bias 7, 3 mantissa bits,
  subnormals, S.1111.111 = NaN, max 448) -- known code values, round trip of every finite
  code, ties to even, and agreement with torch's CPU float8_e4m3fn cast inside the range.
* Hadamard: H H^T = d I and equality with scipy.linalg.hadamard (Sylvester construction).
* Incoherent processing (FlashAttention-3 digest, section 3.5): (Q D H)(K D H)^T / d = Q K^T.
* The whole pre-pass in exact rational arithmetic (fractions.Fraction) on small inputs.
"""
import math
from fractions import Fraction

import numpy as np
import pytest
import scipy.linalg
import torch

import seeded_inputs
from oracle import bf16_to_f64, fp8


def test_e4m3_known_codes():
    dec = fp8.e4m3_decode(np.arange(256, dtype=np.uint8))
    assert dec[0x7E] == 448.0 and dec[0xFE] == -448.0
    assert dec[0x38] == 1.0
    assert dec[0x08] == 2.0 ** -6  # smallest normal
    assert dec[0x01] == 2.0 ** -9  # smallest subnormal
    assert dec[0x07] == 7 * 2.0 ** -9  # largest subnormal
    assert dec[0x00] == 0.0 and math.copysign(1.0, dec[0x80]) == -1.0
    assert np.isnan(dec[0x7F]) and np.isnan(dec[0xFF])
    assert np.sum(np.isnan(dec)) == 2
    pos = dec[:0x7F]
    assert np.all(np.diff(pos) > 0), "non-negative codes must increase with their value"


def test_e4m3_round_trip_and_ties():
    codes = np.array([c for c in range(256) if c not in (0x7F, 0xFF)], dtype=np.uint8)
    assert np.array_equal(fp8.e4m3_encode(fp8.e4m3_decode(codes)), codes)
    pos = fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))
    mids = (pos[:-1] + pos[1:]) / 2
    got = fp8.e4m3_encode(mids)
    lo = np.arange(0x7E)
    want = np.where(lo % 2 == 0, lo, lo + 1)
    assert np.array_equal(got, want), "midpoints must round to the even code"
    eps = np.nextafter(mids, np.inf) - mids
    assert np.array_equal(fp8.e4m3_encode(mids + eps), lo + 1)
    assert np.array_equal(fp8.e4m3_encode(mids - eps), lo)
    assert fp8.e4m3_encode(np.array([1e6, -1e6])).tolist() == [0x7E, 0xFE]


def test_e4m3_matches_torch_in_range():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000) * s for s in (1e-3, 0.1, 1, 30, 200)])
    x = np.clip(x, -448, 448)
    ours = fp8.e4m3_encode(x)
    theirs = torch.from_numpy(x).to(torch.float8_e4m3fn).view(torch.uint8).numpy()
    assert np.array_equal(ours, theirs)


@pytest.mark.parametrize("d", [1, 2, 4, 8, 64, 128, 256])
def test_hadamard(d):
    H = fp8.hadamard(d)
    assert np.array_equal(H @ H.T, d * np.eye(d))
    assert np.array_equal(H, scipy.linalg.hadamard(d).astype(np.float64))


def test_rotation_preserves_scores():
    d = 128
    signs = seeded_inputs.hadamard_signs(d)
    rng = np.random.default_rng(1)
    q, k = rng.standard_normal((50, d)), rng.standard_normal((70, d))
    lhs = fp8.rotate(q, signs) @ fp8.rotate(k, signs).T / d
    np.testing.assert_allclose(lhs, q @ k.T, rtol=0, atol=1e-12)


def test_block_exponent_boundaries():
    assert fp8.block_exponent(0.0) == 0
    assert fp8.block_exponent(448.0) == 0
    assert fp8.block_exponent(np.nextafter(448.0, np.inf)) == 1
    assert fp8.block_exponent(224.0) == -1
    assert fp8.block_exponent(np.nextafter(224.0, np.inf)) == 0
    rng = np.random.default_rng(2)
    for a in np.exp(rng.uniform(-30, 30, 2000)):
        e = fp8.block_exponent(a)
        assert a <= 448.0 * 2.0 ** e and a > 448.0 * 2.0 ** (e - 1)


def _exact_code(x: Fraction) -> int:
    """Nearest e4m3 code by exact rational comparison, ties to even, sign kept."""
    table = [Fraction(float(v)) for v in fp8.e4m3_decode(np.arange(0x7F, dtype=np.uint8))]
    a = min(abs(x), Fraction(448))
    best = min(range(0x7F), key=lambda c: (abs(table[c] - a), c % 2))
    return best | (0x80 if x < 0 else 0)


def test_prepare_exact_small():
    """Rotation, block exponents and codes of the pre-pass equal exact rational arithmetic."""
    inp = seeded_inputs.fp8_inputs(1, 70, 2, 16, seed=9, fraction=0.05)
    signs = seeded_inputs.hadamard_signs(16, seed=3)
    q, k, v = (bf16_to_f64(getattr(inp, n)) for n in "qkv")
    q8, k8, v8, sq, sk, sv = fp8.fp8_prepare(q, k, v, signs)
    H = fp8.hadamard(16)
    for name, x, codes, scales, rot in (("q", q, q8, sq, True), ("k", k, k8, sk, True),
                                        ("v", v, v8, sv, False)):
        for h in range(2):
            for blk, (t0, t1) in enumerate(((0, 64), (64, 70))):
                ex = []
                for t in range(t0, t1):
                    row = [Fraction(float(z)) for z in x[0, t, h]]
                    if rot:
                        row = [sum(int(signs[i]) * int(H[i, j]) * row[i] for i in range(16)) for j in range(16)]
                    ex.append(row)
                amax = max(abs(z) for r in ex for z in r)
                e = 0
                if amax:
                    e = math.ceil(math.log2(amax / 448))
                    while amax > 448 * Fraction(2) ** e:
                        e += 1
                    while amax <= 448 * Fraction(2) ** (e - 1):
                        e -= 1
                want_scale = Fraction(2) ** e / (16 if name == "k" else 1)
                assert Fraction(float(scales[0, h, blk])) == want_scale, (name, h, blk)
                for r, t in zip(ex, range(t0, t1)):
                    want = [_exact_code(z / Fraction(2) ** e) for z in r]
                    assert codes[0, t, h].tolist() == want, (name, h, t)


def test_dequantized_error_bound():
    """Every dequantised value is within half a grid step of the (rotated) input."""
    inp = seeded_inputs.fp8_inputs(1, 128, 4, 128, seed=11)
    signs = seeded_inputs.hadamard_signs(128)
    q, k, v = (bf16_to_f64(getattr(inp, n)) for n in "qkv")
    q8, k8, v8, sq, sk, sv = fp8.fp8_prepare(q, k, v, signs)
    for x, codes, s, rot, extra in ((q, q8, sq, True, 1.0), (k, k8, sk, True, 128.0), (v, v8, sv, False, 1.0)):
        y = fp8.rotate(x, signs) if rot else x
        deq = fp8.dequantize(codes, s) * extra
        blk_scale = np.repeat(s.astype(np.float64) * extra, 64, axis=2).transpose(0, 2, 1)[..., None]
        # relative step of e4m3 is 2**-3 for normals; subnormal step is 2**-9 of the scale
        bound = np.maximum(np.abs(y) * 2.0 ** -4, blk_scale * 2.0 ** -10)
        assert np.all(np.abs(deq - y) <= bound * (1 + 1e-12))
