"""FP8 e4m3 pre-pass of the attention forward pass, written from its definition.

TEST INFRASTRUCTURE ONLY (see the package docstring).

Sources (FlashAttention-3 digest, section 3.5 "FP8 adaptation"; blog article section 4):

* Block quantisation: one scale per block of 64 tokens x d of each head of Q, K and V.
  The scale is a power of two (the blog article, section 4, insists on power-of-two
  scales that are uniform inside a block), so folding it into the scores is exact.
* Incoherent processing: Q and K are multiplied by the same random orthogonal matrix
  M = D H / sqrt(d) before quantising, with D a random +-1 diagonal and H the Sylvester
  Hadamard matrix; (QM)(KM)^T = QK^T.  Here H is kept unnormalised (entries +-1), so
  (Q D H)(K D H)^T = d * Q K^T and the 1/d is folded into K's block scales.  V is not
  rotated.
* e4m3 is the OCP 8-bit floating-point format E4M3 ("fn" variant): 4 exponent bits with
  bias 7, 3 mantissa bits, subnormals, no infinities, S.1111.111 is NaN, largest finite
  magnitude 448.  Encoding rounds to nearest with ties to even and clamps to +-448.

Readings where the pages leave a step open:

* Block exponent e is the smallest integer with amax <= 448 * 2**e (amax = 0 gives e = 0),
  so the block's largest magnitude lands in [224, 448] after scaling.
* Blocks start at token 0 of every (batch, head); a short last block is scaled over its
  valid tokens only.
* A scale must be a normal fp32 power of two, 2**-126 or more: the attention takes each scale
  as the 8-bit exponent of the matrix instruction's scale operand (OCP E8M0), and a denormal
  fp32 has no such exponent.  A block (or tensor) whose exponent would give a smaller scale
  gets the smallest allowed one; its values then land among the e4m3 subnormals or round to
  zero.  The pages never meet this case (their inputs are O(1)).
* The code of an element follows its exact value: an exact zero (also a -0.0 input, or a
  rotated sum that cancels exactly) encodes as +0, and a nonzero value too small for e4m3
  rounds to the zero of its own sign.
* Per-tensor scaling, the usual practice that the digest's section 3.5 contrasts with block
  quantisation (and the baseline of its Table 3 ablation), uses one exponent for a whole
  tensor, chosen by the same rule from the tensor's largest magnitude; the scale arrays keep
  their per-block shape with every entry equal.
* Rotary position embedding before the rotation (the digest's section 3.5 fuses the pre-pass
  into the rotary embedding that precedes attention; the guijiagi overview's "fusion with
  RoPE" paragraph).  The pages do not define the embedding, so the original RoFormer form is
  read: features (2i, 2i+1) of the token at position m (counted from its sequence's first
  token) are rotated by the angle whose cosine and sine the caller tabulates in fp32 at
  [m, i].  Each output is formed as a rotary kernel working in fp32 forms it -- x0*c - x1*s
  and x0*s + x1*c, every product and sum rounded to fp32 -- and rounded to bf16 (nearest,
  ties to even), i.e. the bf16 tensor an unfused rotary kernel would hand on; the pre-pass
  then proceeds on it.
* The Hadamard sums are formed exactly (fp64 sums of bf16 values with +-1 weights are exact
  unless one row spans more than 2**38 in magnitude), so the code chosen for each element is
  the round-to-nearest-even of the exact rotated value.
"""
from __future__ import annotations

import math

import numpy as np

BLOCK = 64
E4M3_MAX = 448.0


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    """Value of each e4m3fn code (uint8) as float64; NaN codes decode to NaN."""
    c = np.asarray(codes, dtype=np.uint8).astype(np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = c & 0x7
    mag = np.where(e == 0, (m / 8.0) * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (m == 7), np.nan, mag)
    return sign * mag


# All non-negative finite magnitudes, indexed by their code 0x00..0x7E (increasing).
_POS_TABLE = e4m3_decode(np.arange(0x7F, dtype=np.uint8))


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Nearest e4m3fn code to each float64 value, ties to the even code, clamped to +-448.

    Implemented as a search over the table of representable magnitudes, which is the
    format's definition rather than a bit trick.
    """
    x = np.asarray(x, dtype=np.float64)
    if np.any(np.isnan(x)):
        raise ValueError("e4m3_encode got NaN")
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.searchsorted(_POS_TABLE, a, side="left")  # first table entry >= a
    hi = np.minimum(hi, 0x7E)
    lo = np.maximum(hi - 1, 0)
    d_lo = a - _POS_TABLE[lo]
    d_hi = _POS_TABLE[hi] - a
    pick_hi = (d_hi < d_lo) | ((d_hi == d_lo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo)
    code = np.where(a == _POS_TABLE[hi], hi, code)
    # the sign is kept, also when the magnitude rounds to zero (IEEE-style signed zero)
    return (code | np.where(np.signbit(x), 0x80, 0)).astype(np.uint8)


def hadamard(d: int) -> np.ndarray:
    """Unnormalised Sylvester Hadamard matrix: H[i, j] = (-1)**popcount(i & j)."""
    if d <= 0 or d & (d - 1):
        raise ValueError("d must be a power of two")
    i = np.arange(d)
    pc = np.vectorize(lambda x: bin(int(x)).count("1"))(i[:, None] & i[None, :])
    return np.where(pc % 2 == 0, 1.0, -1.0)


def block_exponent(amax: float) -> int:
    """Smallest integer e with amax <= 448 * 2**e; 0 for amax == 0."""
    if amax == 0.0:
        return 0
    m, ex = math.frexp(amax)  # amax = m * 2**ex with 0.5 <= m < 1
    # 448 = 0.875 * 2**9, and m / 0.875 lies in (0.57, 1.15)
    return ex - 9 if m <= 0.875 else ex - 8


def rotate(x: np.ndarray, signs: np.ndarray | None) -> np.ndarray:
    """x D H along the last axis (fp64).  signs=None means no rotation."""
    x = np.asarray(x, dtype=np.float64)
    if signs is None:
        return x
    d = x.shape[-1]
    return (x * np.asarray(signs, dtype=np.float64)) @ hadamard(d)


# Smallest exponent of a normal fp32 (and of a usable E8M0 scale operand).
SCALE_EXP_MIN = -126


def _nblocks(N: int, block: int) -> int:
    return -(-N // block)


def _encode_with(y: np.ndarray, exps: np.ndarray, block: int) -> np.ndarray:
    """e4m3 codes of y [B, N, H, d] divided by 2**exps[b, h, token // block]."""
    B, N, H, d = y.shape
    codes = np.empty(y.shape, dtype=np.uint8)
    for b in range(B):
        for h in range(H):
            for j in range(_nblocks(N, block)):
                t0, t1 = j * block, min(N, (j + 1) * block)
                # + 0.0 clears the sign of an exact zero (a -0.0 input, or a rotated sum that
                # is exactly zero), so the code follows the value: exact zero -> +0.
                codes[b, t0:t1, h, :] = e4m3_encode(np.ldexp(y[b, t0:t1, h, :], -int(exps[b, h, j])) + 0.0)
    return codes


def quantize_blocks(y: np.ndarray, block: int = BLOCK, e_floor: int = SCALE_EXP_MIN):
    """Per-(batch, head, 64-token block) power-of-two scaling and e4m3 encoding.

    y: [B, N, H, d] float64.  Returns (codes uint8 [B,N,H,d], exponents int [B,H,nblk]); each
    exponent is the block's own, raised to e_floor if it is smaller.
    """
    B, N, H, d = y.shape
    exps = np.zeros((B, H, _nblocks(N, block)), dtype=np.int64)
    for b in range(B):
        for h in range(H):
            for j in range(exps.shape[2]):
                blk = y[b, j * block:min(N, (j + 1) * block), h, :]
                exps[b, h, j] = max(block_exponent(float(np.max(np.abs(blk))) if blk.size else 0.0), e_floor)
    return _encode_with(y, exps, block), exps


def quantize_tensor(y: np.ndarray, block: int = BLOCK, e_floor: int = SCALE_EXP_MIN):
    """Per-tensor power-of-two scaling: one exponent, from the largest magnitude of all of y,
    for every block.  Same outputs as :func:`quantize_blocks`."""
    B, N, H, d = y.shape
    e = max(block_exponent(float(np.max(np.abs(y))) if y.size else 0.0), e_floor)
    exps = np.full((B, H, _nblocks(N, block)), e, dtype=np.int64)
    return _encode_with(y, exps, block), exps


def fp8_prepare(q, k, v, signs: np.ndarray | None, block: int = BLOCK, per_tensor: bool = False):
    """The full pre-pass on fp64 copies of the bf16 inputs ([B, N, H, d] each).

    Returns q8, k8, v8 (uint8 e4m3 codes) and q_scale, k_scale, v_scale (float32
    [B, H, nblk], powers of two).  With signs given, Q and K are rotated by D H and K's
    scales carry the extra 1/d.  per_tensor selects one scale per tensor instead of one per
    block.  Every scale is 2**-126 or more.
    """
    d = np.shape(q)[-1]
    shift_k = int(math.log2(d)) if signs is not None else 0
    quant = quantize_tensor if per_tensor else quantize_blocks
    q8, eq = quant(rotate(q, signs), block)
    k8, ek = quant(rotate(k, signs), block, SCALE_EXP_MIN + shift_k)
    v8, ev = quant(np.asarray(v, dtype=np.float64), block)
    to_scale = lambda e: np.ldexp(np.ones(e.shape, dtype=np.float32), e.astype(np.int32))
    return q8, k8, v8, to_scale(eq), to_scale(ek - shift_k), to_scale(ev)


def bf16_round(x: np.ndarray) -> np.ndarray:
    """float32 -> nearest bfloat16 value (ties to the even significand), returned as float32.
    Finite inputs only: the dropped 16 bits decide the rounding of the kept 16."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    keep_lsb = (u >> 16) & 1
    r = ((u + 0x7FFF + keep_lsb) >> 16) << 16
    return r.astype(np.uint32).view(np.float32)


def rope(x: np.ndarray, cos: np.ndarray, sin: np.ndarray, positions: np.ndarray) -> np.ndarray:
    """Rotary embedding of x [..., T, H, d] (fp64 copies of bf16 values) at the given token
    positions [T] (broadcast over leading axes), with fp32 tables cos, sin [>= max position + 1,
    d/2]; returns the bf16 results as float64."""
    x = np.asarray(x, dtype=np.float64)
    x0 = x[..., 0::2].astype(np.float32)  # exact: bf16 values are fp32 values
    x1 = x[..., 1::2].astype(np.float32)
    c = np.asarray(cos, dtype=np.float32)[positions][:, None, :]  # [T, 1, d/2]
    s = np.asarray(sin, dtype=np.float32)[positions][:, None, :]
    r0 = (x0 * c) - (x1 * s)  # float32 operations, each rounded to nearest
    r1 = (x0 * s) + (x1 * c)
    out = np.empty(x.shape, dtype=np.float64)
    out[..., 0::2] = bf16_round(r0)
    out[..., 1::2] = bf16_round(r1)
    return out


def rope_prepare(q, k, v, cos, sin, signs: np.ndarray | None, per_tensor: bool = False, cu_seqlens=None,
                 max_seqlen: int | None = None):
    """The pre-pass with the rotary embedding first: Q and K are embedded at their positions
    within their sequences, V is not; then :func:`fp8_prepare` (dense [B, N, H, d]) or
    :func:`fp8_prepare_varlen` (packed [T, H, d])."""
    if cu_seqlens is None:
        N = np.shape(q)[1]
        pos = np.arange(N)
        return fp8_prepare(rope(q, cos, sin, pos), rope(k, cos, sin, pos), v, signs, per_tensor=per_tensor)
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    pos = np.concatenate([np.arange(cu[b + 1] - cu[b]) for b in range(len(cu) - 1)]).astype(np.int64)
    return fp8_prepare_varlen(rope(q, cos, sin, pos), rope(k, cos, sin, pos), v, cu, max_seqlen, signs,
                              per_tensor=per_tensor)


def fp8_prepare_varlen(q, k, v, cu_seqlens, max_seqlen: int, signs: np.ndarray | None, block: int = BLOCK,
                       per_tensor: bool = False):
    """The pre-pass on packed sequences: q [T, Hq, d], k and v [T, Hkv, d] (fp64 copies of the
    bf16 inputs); sequence b holds tokens cu_seqlens[b] .. cu_seqlens[b+1]-1.

    Blocks start at every sequence's first token, so each sequence is quantised as the dense
    pre-pass would quantise it alone.  Scales are float32 [nseq, H, ceil(max_seqlen/64)].  With
    per-block scales, entries past a sequence's last block are NaN (not defined); with
    per_tensor, one exponent comes from the largest magnitude of the whole packed tensor and
    every entry holds its scale.
    """
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    nseq = len(cu) - 1
    d = np.shape(q)[-1]
    shift_k = int(math.log2(d)) if signs is not None else 0
    nblk = _nblocks(max_seqlen, block)
    out_codes, out_scales = [], []
    for x, rot, floor, shift in ((q, True, SCALE_EXP_MIN, 0), (k, True, SCALE_EXP_MIN + shift_k, shift_k),
                                 (v, False, SCALE_EXP_MIN, 0)):
        y = rotate(x, signs) if rot else np.asarray(x, dtype=np.float64)
        T, H, _ = y.shape
        codes = np.empty(y.shape, dtype=np.uint8)
        exps = np.full((nseq, H, nblk), np.nan)
        e_tensor = max(block_exponent(float(np.max(np.abs(y))) if y.size else 0.0), floor)
        for b in range(nseq):
            seq = y[None, cu[b]:cu[b + 1]]  # [1, n_b, H, d]
            if per_tensor:
                e = np.full((1, H, _nblocks(seq.shape[1], block)), e_tensor, dtype=np.int64)
                c = _encode_with(seq, e, block)
                exps[b] = e_tensor
            else:
                c, e = quantize_blocks(seq, block, floor)
                exps[b, :, :e.shape[2]] = e[0]
            codes[cu[b]:cu[b + 1]] = c[0]
        out_codes.append(codes)
        out_scales.append(np.where(np.isnan(exps), np.float32(np.nan),
                                   np.ldexp(np.float32(1.0), np.nan_to_num(exps - shift).astype(np.int32))
                                   ).astype(np.float32))
    return (*out_codes, *out_scales)


def dequantize_varlen(codes: np.ndarray, scales: np.ndarray, cu_seqlens, block: int = BLOCK) -> np.ndarray:
    """codes [T,H,d] of packed sequences with scales [nseq,H,nblk] -> float64 [T,H,d] (exact)."""
    cu = np.asarray(cu_seqlens, dtype=np.int64)
    out = np.empty(codes.shape, dtype=np.float64)
    for b in range(len(cu) - 1):
        seq = codes[None, cu[b]:cu[b + 1]]
        nb = _nblocks(seq.shape[1], block)
        out[cu[b]:cu[b + 1]] = dequantize(seq, scales[b:b + 1, :, :nb], block)[0]
    return out


def dequantize(codes: np.ndarray, scales: np.ndarray, block: int = BLOCK) -> np.ndarray:
    """codes [B,N,H,d] with scales [B,H,nblk] -> float64 [B,N,H,d] (exact)."""
    B, N, H, d = codes.shape
    tok_blk = np.arange(N) // block
    s = np.asarray(scales, dtype=np.float64)[:, :, tok_blk]  # [B, H, N]
    return e4m3_decode(codes) * s.transpose(0, 2, 1)[..., None]
