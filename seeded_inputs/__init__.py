"""Seeded synthetic inputs shared by the oracle tests, the GPU parity tests and the benchmark.

This module only draws random numbers and rounds them to the storage formats the
kernels take (bf16, fp16).  It holds none of the attention arithmetic, so both the
CPU oracle and the HIP path can consume its output without sharing any of the
method's code.

Workloads (shapes follow the attention problem statement of the FlashAttention-3
pages, "3.1 computation definition" and the Table-2 ablation shape):

* dense  : Q [B, N, Hq, d], K/V [B, N, Hkv, d]
* varlen : Q [T, Hq, d],    K/V [T, Hkv, d] with int32 cu_seqlens [nseq + 1]

Every tensor is drawn as i.i.d. N(0, 1) float32 with ``numpy.random.default_rng(seed)``
in the order Q, K, V and then rounded to the storage dtype with round-to-nearest-even.
"""
from __future__ import annotations

from dataclasses import dataclass, field

import numpy as np

__all__ = [
    "f32_to_bf16_bits",
    "bf16_bits_to_f32",
    "AttnInputs",
    "dense_inputs",
    "varlen_lengths",
    "varlen_inputs",
    "outlier_channels",
    "fp8_inputs",
    "mixture_inputs",
    "hadamard_signs",
    "rope_tables",
    "output_gradient",
    "CONFIGS",
]


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 to bfloat16 (round to nearest, ties to even); return the uint16 bit patterns."""
    x = np.ascontiguousarray(x, dtype=np.float32)
    if not np.all(np.isfinite(x)):
        raise ValueError("generator produced a non-finite value")
    u = x.view(np.uint32).astype(np.uint64)
    lsb = (u >> 16) & 1
    r = (u + 0x7FFF + lsb) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns to float32."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32)


@dataclass
class AttnInputs:
    """One seeded attention problem.

    ``q``, ``k``, ``v`` hold storage bit patterns: uint16 for bf16/fp16.  ``dtype`` is
    "bf16" or "fp16".  ``cu_seqlens`` is None for dense inputs.  ``window`` > 0 (with causal)
    asks for a sliding window: query i sees keys i-window+1 .. i.
    """

    q: np.ndarray
    k: np.ndarray
    v: np.ndarray
    dtype: str
    B: int
    N: int
    Hq: int
    Hkv: int
    d: int
    causal: bool
    cu_seqlens: np.ndarray | None = None
    seed: int = 0
    meta: dict = field(default_factory=dict)
    window: int = 0

    @property
    def alpha(self) -> float:
        return 1.0 / float(np.sqrt(self.d))

    @property
    def total_tokens(self) -> int:
        return int(self.cu_seqlens[-1]) if self.cu_seqlens is not None else self.B * self.N

    def seqlens(self) -> np.ndarray:
        if self.cu_seqlens is None:
            return np.full(self.B, self.N, dtype=np.int64)
        return np.diff(self.cu_seqlens.astype(np.int64))

    def flops(self) -> float:
        """4 * Hq * d * (sum over sequences of n^2), halved when causal; with a window W the
        causal count n^2/2 loses the (n-W)^2/2 pairs at least W apart (same convention)."""
        n = self.seqlens().astype(np.float64)
        if self.causal and self.window > 0:
            far = np.maximum(n - self.window, 0.0)
            return 4.0 * self.Hq * self.d * float(np.sum(n * n - far * far)) / 2.0
        f = 4.0 * self.Hq * self.d * float(np.sum(n * n))
        return f / 2.0 if self.causal else f

    def widened(self, name: str) -> np.ndarray:
        """float32 view of a stored tensor (exact for bf16 and fp16)."""
        a = getattr(self, name)
        if self.dtype == "bf16":
            return bf16_bits_to_f32(a)
        return a.view(np.float16).astype(np.float32)


def _to_storage(x: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return f32_to_bf16_bits(x)
    if dtype == "fp16":
        return np.ascontiguousarray(x.astype(np.float16)).view(np.uint16)
    raise ValueError(f"unknown storage dtype {dtype!r}")


def dense_inputs(B: int, N: int, Hq: int, d: int, *, Hkv: int | None = None, causal: bool = False,
                 seed: int = 0, dtype: str = "bf16") -> AttnInputs:
    """Dense [B, N, H, d] tensors, i.i.d. N(0,1), drawn in the order Q, K, V."""
    Hkv = Hq if Hkv is None else Hkv
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, Hq, d), dtype=np.float32)
    k = rng.standard_normal((B, N, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((B, N, Hkv, d), dtype=np.float32)
    return AttnInputs(_to_storage(q, dtype), _to_storage(k, dtype), _to_storage(v, dtype), dtype,
                      B, N, Hq, Hkv, d, causal, None, seed)


def varlen_lengths(rng: np.random.Generator, nseq: int, lo: int, hi: int) -> np.ndarray:
    """Sequence lengths drawn uniformly from the integers lo..hi inclusive."""
    return rng.integers(lo, hi + 1, nseq).astype(np.int64)


def varlen_inputs(lengths, Hq: int, Hkv: int, d: int, *, causal: bool = True, seed: int = 0,
                  dtype: str = "bf16", rng: np.random.Generator | None = None) -> AttnInputs:
    """Packed [T, H, d] tensors with int32 cu_seqlens; Q, K, V drawn after the lengths."""
    rng = np.random.default_rng(seed) if rng is None else rng
    lengths = np.asarray(lengths, dtype=np.int64)
    cu = np.zeros(len(lengths) + 1, dtype=np.int32)
    cu[1:] = np.cumsum(lengths)
    T = int(cu[-1])
    q = rng.standard_normal((T, Hq, d), dtype=np.float32)
    k = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    v = rng.standard_normal((T, Hkv, d), dtype=np.float32)
    return AttnInputs(_to_storage(q, dtype), _to_storage(k, dtype), _to_storage(v, dtype), dtype,
                      len(lengths), int(lengths.max()) if len(lengths) else 0, Hq, Hkv, d, causal,
                      cu, seed)


def outlier_channels(rng: np.random.Generator, H: int, d: int, fraction: float = 0.001) -> np.ndarray:
    """Indices (into the flattened H*d feature axis) of the channels scaled up as outliers."""
    count = max(1, int(round(fraction * H * d)))
    return np.sort(rng.choice(H * d, size=count, replace=False))


def fp8_inputs(B: int, N: int, H: int, d: int, *, seed: int = 5, outlier_scale: float = 20.0,
               fraction: float = 0.001, independent_channels: bool = False) -> AttnInputs:
    """bf16 Q, K, V i.i.d. N(0,1) with a fraction of the H*d feature channels scaled by
    ``outlier_scale`` before the bf16 rounding.  Channel indices are drawn after Q, K, V: one
    set shared by Q, K and V, or (``independent_channels``) one draw per tensor in the order
    Q, K, V."""
    rng = np.random.default_rng(seed)
    q = rng.standard_normal((B, N, H, d), dtype=np.float32)
    k = rng.standard_normal((B, N, H, d), dtype=np.float32)
    v = rng.standard_normal((B, N, H, d), dtype=np.float32)
    shared = outlier_channels(rng, H, d, fraction)
    chans = []
    for t in (q, k, v):
        ch = outlier_channels(rng, H, d, fraction) if independent_channels and chans else shared
        chans.append(ch)
        flat = t.reshape(B, N, H * d)
        flat[:, :, ch] *= np.float32(outlier_scale)
    inp = AttnInputs(f32_to_bf16_bits(q), f32_to_bf16_bits(k), f32_to_bf16_bits(v), "bf16",
                     B, N, H, H, d, False, None, seed)
    inp.meta["outlier_channels"] = chans[0] if not independent_channels else chans
    return inp


def mixture_inputs(B: int, N: int, H: int, d: int, *, seed: int, outlier_prob: float = 0.001,
                   outlier_std: float = 10.0, dtype: str = "bf16") -> AttnInputs:
    """Q, K, V whose elements are i.i.d. N(0, 1) + N(0, outlier_std**2) * Bernoulli(outlier_prob)
    (the outlier model of the FlashAttention-3 paper's numerical-error experiment, section 4.3),
    rounded to ``dtype``.  Per tensor, in the order Q, K, V: the N(0, 1) part, then uniforms
    u (the element is an outlier when u < outlier_prob), then the N(0, 1) draws scaled by
    outlier_std."""
    rng = np.random.default_rng(seed)
    out = []
    for _ in range(3):
        x = rng.standard_normal((B, N, H, d), dtype=np.float32)
        hit = rng.random((B, N, H, d), dtype=np.float32) < np.float32(outlier_prob)
        x += np.where(hit, rng.standard_normal((B, N, H, d), dtype=np.float32) * np.float32(outlier_std),
                      np.float32(0.0))
        out.append(_to_storage(x, dtype))
    inp = AttnInputs(out[0], out[1], out[2], dtype, B, N, H, H, d, False, None, seed)
    inp.meta["outlier_prob"] = outlier_prob
    inp.meta["outlier_std"] = outlier_std
    return inp


def output_gradient(inp: AttnInputs, seed: int) -> np.ndarray:
    """dO for a backward pass: i.i.d. N(0, 1) in the layout of Q (= O), rounded to inp.dtype."""
    rng = np.random.default_rng(seed)
    return _to_storage(rng.standard_normal(inp.q.shape, dtype=np.float32), inp.dtype)


def rope_tables(positions: int, d: int, base: float = 10000.0):
    """fp32 cos and sin tables [positions, d/2] of RoFormer's angles m * base^(-2i/d), formed in
    float64 and rounded once to float32 (inputs of the fused rotary pre-pass)."""
    ang = np.arange(positions, dtype=np.float64)[:, None] * base ** (-np.arange(0, d, 2, dtype=np.float64) / d)
    return np.cos(ang).astype(np.float32), np.sin(ang).astype(np.float32)


def hadamard_signs(d: int, seed: int = 55) -> np.ndarray:
    """The random diagonal of +-1 entries used for incoherent processing (int8, length d)."""
    rng = np.random.default_rng(seed)
    return np.where(rng.integers(0, 2, d) == 0, 1, -1).astype(np.int8)


# The five workloads: (name, builder).  Seeds: 1..5 in order; Hadamard signs from seed 55.
def _c1():
    return dense_inputs(1, 128, 2, 64, seed=1)


def _c2(N: int):
    return dense_inputs(16384 // N, N, 16, 128, seed=2)


def _c3(d: int):
    return dense_inputs(2, 8192, 16, d, causal=True, seed=3)


def _c4():
    rng = np.random.default_rng(4)
    lengths = varlen_lengths(rng, 8, 256, 8192)
    return varlen_inputs(lengths, 32, 8, 128, causal=True, seed=4, rng=rng)


def _c5():
    return fp8_inputs(2, 8192, 16, 128, seed=5)


CONFIGS = {
    "mha_b1_h2_n128_d64": _c1,
    **{f"mha_n{N}_b{16384 // N}_h16_d128": (lambda N=N: _c2(N)) for N in (512, 1024, 2048, 4096, 8192, 16384)},
    **{f"causal_b2_h16_n8192_d{d}": (lambda d=d: _c3(d)) for d in (64, 128, 256)},
    "gqa_varlen_causal_hq32_hkv8_d128": _c4,
    "fp8_b2_h16_n8192_d128": _c5,
}
