"""CPU oracle for exact attention and for the FP8 pre-pass.

TEST INFRASTRUCTURE ONLY.  Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline
leg of ``bench.py`` may import this package.  The product path (``exact_attention_76_amd``)
never imports it and never falls back to it.

* :func:`attention` / :func:`attention_rows` -- the plain fp64 definition of attention
  (FlashAttention-3 digest, section 3.1; LSE from the Algorithm-1 epilogue in section 3.2),
  implemented in C (``attn_oracle.c``) as a two-pass loop nest per query row.
* :mod:`oracle.fp8` -- the FP8 e4m3 pre-pass: random +-1 diagonal times Hadamard rotation of
  Q and K, per-block power-of-two scales, e4m3 encoding (digest section 3.5).
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "attn_oracle.c")
_LIB = os.path.join(_HERE, "liboracle.so")
_lib = None


def compile_source(src: str, out: str) -> str:
    """Compile one C source of the oracle into a shared library (gcc, -O2, OpenMP)."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-fopenmp", "-shared", "-fPIC", "-std=c11", "-o", tmp, src, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile attn_oracle.c into oracle/liboracle.so."""
    if force or not os.path.exists(_LIB):
        compile_source(_SRC, _LIB)
    return _LIB


class OracleLib:
    """ctypes handle on one build of attn_oracle.c (the tests also build altered copies)."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        P = ctypes.c_void_p
        I64 = ctypes.c_int64
        lib.oracle_attention_rows.argtypes = [P, P, P, I64, I64, I64, P, I64, ctypes.c_int, I64,
                                              ctypes.c_double, P, P, I64, P, P]
        lib.oracle_attention_rows.restype = ctypes.c_int
        lib.oracle_attention.argtypes = [P, P, P, I64, I64, I64, P, I64, ctypes.c_int, I64,
                                         ctypes.c_double, P, P]
        lib.oracle_attention.restype = ctypes.c_int
        lib.oracle_num_threads.restype = ctypes.c_int
        lib.oracle_set_num_threads.argtypes = [ctypes.c_int]
        lib.oracle_set_num_threads.restype = None
        self.lib = lib

    def num_threads(self) -> int:
        return int(self.lib.oracle_num_threads())

    def set_num_threads(self, n: int) -> None:
        self.lib.oracle_set_num_threads(int(n))

    def attention(self, q, k, v, *, causal: bool = False, alpha: float | None = None, cu_seqlens=None,
                  window: int = 0):
        """fp64 attention over every row.  ``window`` > 0: query i also needs keys j > i - window.

        Dense: q [B,N,Hq,d], k/v [B,N,Hkv,d] -> (o [B,N,Hq,d], lse [B,Hq,N]).
        Varlen: q [T,Hq,d], k/v [T,Hkv,d], cu_seqlens [nseq+1] -> (o [T,Hq,d], lse [Hq,T]).
        ``alpha`` defaults to 1/sqrt(d).
        """
        dense = cu_seqlens is None
        shape = np.shape(q)
        qp, kp, vp, cu = _pack(q, k, v, cu_seqlens)
        T, Hq, d = qp.shape
        Hkv = kp.shape[1]
        alpha = 1.0 / np.sqrt(d) if alpha is None else float(alpha)
        o = np.empty((T, Hq, d), dtype=np.float64)
        lse = np.empty((Hq, T), dtype=np.float64)
        rc = self.lib.oracle_attention(_ptr(qp), _ptr(kp), _ptr(vp), Hq, Hkv, d, _ptr(cu), len(cu) - 1,
                                       int(bool(causal)), int(window), alpha, _ptr(o), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        if dense:
            B, N = shape[:2]
            return o.reshape(B, N, Hq, d), np.ascontiguousarray(lse.reshape(Hq, B, N).transpose(1, 0, 2))
        return o, lse

    def attention_rows(self, q, k, v, heads, tokens, *, causal: bool = False, alpha: float | None = None,
                       cu_seqlens=None, window: int = 0):
        """fp64 attention for selected rows only.

        ``tokens`` are packed token indices (dense: b*N + i).  Returns (o [n, d], lse [n]).
        """
        qp, kp, vp, cu = _pack(q, k, v, cu_seqlens)
        T, Hq, d = qp.shape
        Hkv = kp.shape[1]
        alpha = 1.0 / np.sqrt(d) if alpha is None else float(alpha)
        heads = np.ascontiguousarray(heads, dtype=np.int64)
        tokens = np.ascontiguousarray(tokens, dtype=np.int64)
        if heads.shape != tokens.shape or heads.ndim != 1:
            raise ValueError("heads and tokens must be 1-D and of equal length")
        o = np.empty((len(heads), d), dtype=np.float64)
        lse = np.empty(len(heads), dtype=np.float64)
        rc = self.lib.oracle_attention_rows(_ptr(qp), _ptr(kp), _ptr(vp), Hq, Hkv, d, _ptr(cu),
                                            len(cu) - 1, int(bool(causal)), int(window), alpha, _ptr(heads),
                                            _ptr(tokens), len(heads), _ptr(o), _ptr(lse))
        if rc != 0:
            raise ValueError("oracle rejected its arguments")
        return o, lse


def _load() -> OracleLib:
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB):
            build()
        _lib = OracleLib(_LIB)
    return _lib


def _ptr(a: np.ndarray):
    return a.ctypes.data_as(ctypes.c_void_p)


def _pack(q, k, v, cu_seqlens):
    """Bring dense [B,N,H,d] or packed [T,H,d] fp64 inputs to the packed form + int64 offsets."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    if cu_seqlens is None:
        if q.ndim != 4:
            raise ValueError("dense inputs are [B, N, H, d]")
        B, N = q.shape[:2]
        cu = np.arange(B + 1, dtype=np.int64) * N
        q = q.reshape(B * N, *q.shape[2:])
        k = k.reshape(B * N, *k.shape[2:])
        v = v.reshape(B * N, *v.shape[2:])
    else:
        cu = np.asarray(cu_seqlens, dtype=np.int64)
        if q.ndim != 3:
            raise ValueError("varlen inputs are [T, H, d]")
    q = np.ascontiguousarray(q)
    k = np.ascontiguousarray(k)
    v = np.ascontiguousarray(v)
    if k.shape != v.shape or q.shape[0] != k.shape[0] or q.shape[2] != k.shape[2]:
        raise ValueError("q/k/v shapes disagree")
    if cu[0] != 0 or cu[-1] != q.shape[0] or np.any(np.diff(cu) < 0):
        raise ValueError("cu_seqlens must start at 0, be non-decreasing and end at T")
    return q, k, v, cu


def num_threads() -> int:
    return _load().num_threads()


def set_num_threads(n: int) -> None:
    """OpenMP threads of the following oracle calls (the benchmark's one-core figure uses 1)."""
    _load().set_num_threads(n)


def attention(q, k, v, **kw):
    """See :meth:`OracleLib.attention`."""
    return _load().attention(q, k, v, **kw)


def attention_rows(q, k, v, heads, tokens, **kw):
    """See :meth:`OracleLib.attention_rows`."""
    return _load().attention_rows(q, k, v, heads, tokens, **kw)


def bf16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of bfloat16 bit patterns (uint16) to float64."""
    b = np.ascontiguousarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def fp16_to_f64(bits: np.ndarray) -> np.ndarray:
    """Exact widening of IEEE half bit patterns (uint16) to float64."""
    return np.ascontiguousarray(bits, dtype=np.uint16).view(np.float16).astype(np.float64)


def widen(bits: np.ndarray, dtype: str) -> np.ndarray:
    if dtype == "bf16":
        return bf16_to_f64(bits)
    if dtype == "fp16":
        return fp16_to_f64(bits)
    raise ValueError(dtype)


def error_metrics(o_test, o_ref, lse_test=None, lse_ref=None) -> dict:
    """max-abs and RMSE over O (the accuracy measures of the digest's section 7.1 / Table 3),
    and the max-abs LSE error."""
    diff = np.asarray(o_test, dtype=np.float64) - np.asarray(o_ref, dtype=np.float64)
    out = {"max_abs": float(np.max(np.abs(diff))) if diff.size else 0.0,
           "rmse": float(np.sqrt(np.mean(diff * diff))) if diff.size else 0.0}
    if lse_test is not None:
        dl = np.asarray(lse_test, dtype=np.float64) - np.asarray(lse_ref, dtype=np.float64)
        out["lse_max_abs"] = float(np.max(np.abs(dl))) if dl.size else 0.0
    return out
