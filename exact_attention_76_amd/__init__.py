"""Python binding of libattn -- the fused exact-attention forward pass for MI355X (gfx950).

Argument marshalling only: every step of the computation runs in the HIP kernels of
``libattn.so`` (sources under ``csrc/``, C ABI in ``include/attn.h``).  PyTorch supplies device
memory and streams.  There is no fallback: if the library cannot be loaded, every call raises.

Entry points carry the names of the C ABI:

* :func:`attn_fwd` -- O and LSE of exact attention (bf16 / fp16 / fp8-e4m3 inputs; dense or
  packed variable-length; causal or not; grouped-query heads).
* :func:`attn_fwd_window` -- the same, causal, inside a sliding window of W keys.
* :func:`attn_bwd` -- dQ, dK, dV of attn_fwd's output (16-bit inputs); with ``window`` it calls
  ``attn_bwd_window`` (the C entry point of the same name).
* :func:`attn_bwd_noalloc` -- attn_bwd without a workspace argument, for callers that cannot
  allocate device memory (the library's static per-GPU workspace).
* :func:`attn_fp8_prepare` -- Hadamard rotation + per-block power-of-two e4m3 quantisation.
* :func:`attn_fp8_prepare_ex` -- the same for packed sequences too, with per-block or per-tensor
  scales.
* :func:`attn_strerror` -- text of a status code.

Helpers :func:`attention` and :func:`fp8_prepare` allocate the outputs and call the above.
"""
from __future__ import annotations

import ctypes
import json
import os
import re

import torch

__all__ = ["AttnError", "check_cu_seqlens", "attn_fwd", "attn_fwd_window", "attn_bwd", "attn_bwd_window", "attn_bwd_noalloc",
           "attention_backward", "attn_fp8_prepare", "attn_fp8_prepare_ex", "attn_strerror", "attention",
           "fp8_prepare", "load_library", "LIB_PATH", "ATTN_BF16", "ATTN_FP16", "ATTN_FP8_E4M3",
           "ATTN_FP8_SCALE_BLOCK", "ATTN_FP8_SCALE_TENSOR"]

_PKG = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG, "libattn.so")
HEADER = os.path.join(os.path.dirname(_PKG), "include", "attn.h")

ATTN_BF16, ATTN_FP16, ATTN_FP8_E4M3 = 0, 1, 2
ATTN_OK, ATTN_ERR_INVALID, ATTN_ERR_UNSUPPORTED, ATTN_ERR_ALIGN, ATTN_ERR_HIP = 0, -1, -2, -3, -4
ATTN_ERR_TOO_LARGE = -5
ATTN_BWD_NOALLOC_MAX_ROWS = 1 << 22
ATTN_FP8_SCALE_BLOCK, ATTN_FP8_SCALE_TENSOR = 0, 1

_lib = None


class AttnError(RuntimeError):
    def __init__(self, status: int, what: str):
        super().__init__(f"{what}: status {status} ({attn_strerror(status)})")
        self.status = status


def check_build_record() -> None:
    """Raise unless libattn.so was built from the sources now on disk: build() records the sha256
    of every source file (and the extra compiler arguments) beside the library."""
    from . import build as _build

    try:
        with open(_build.RECORD) as f:
            built = json.load(f)
    except (OSError, ValueError) as e:
        raise OSError(f"{LIB_PATH} has no readable source record ({_build.RECORD}): rebuild it "
                      "with exact_attention_76_amd/build.py") from e
    now = _build.source_record()
    stale = sorted(set(built.get("sources", {}).items()) ^ set(now["sources"].items()))
    if stale or built.get("extra_flags", "") != now["extra_flags"]:
        what = sorted({name for name, _ in stale}) or [f"compiler arguments {built.get('extra_flags')!r}"]
        raise OSError(f"{LIB_PATH} was not built from the sources on disk (differs in {what}): rebuild it "
                      "with exact_attention_76_amd/build.py")


def load_library(build_if_missing: bool = True):
    """Load libattn.so; compile it first only when no built library exists.  A library built
    from other sources than those on disk is refused (see check_build_record)."""
    global _lib
    if _lib is not None:
        return _lib
    if not os.path.exists(LIB_PATH):
        if not build_if_missing:
            raise OSError(f"{LIB_PATH} is not built")
        from . import build as _build

        _build.build()
    check_build_record()
    lib = ctypes.CDLL(LIB_PATH)
    P, I, F = ctypes.c_void_p, ctypes.c_int, ctypes.c_float
    lib.attn_fwd.argtypes = [P, P, P, P, P, I, I, I, I, P, I, I, F, I, P, P, P, P]
    lib.attn_fwd.restype = I
    lib.attn_fwd_window.argtypes = [P, P, P, P, P, I, I, I, I, P, I, I, F, I, P, P, P, P]
    lib.attn_fwd_window.restype = I
    lib.attn_bwd.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, P, I, I, F, I, P]
    lib.attn_bwd.restype = I
    lib.attn_bwd_window.argtypes = [P, P, P, P, P, P, P, P, P, P, I, I, I, I, P, I, I, F, I, P]
    lib.attn_bwd_window.restype = I
    lib.attn_bwd_noalloc.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, P, I, I, F, I, P]
    lib.attn_bwd_noalloc.restype = I
    lib.attn_bwd_workspace_bytes.argtypes = [I, I, I]
    lib.attn_bwd_workspace_bytes.restype = ctypes.c_size_t
    lib.attn_fp8_prepare.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, I, P, P]
    lib.attn_fp8_prepare.restype = I
    lib.attn_fp8_prepare_ex.argtypes = [P, P, P, P, P, P, P, P, P, I, I, I, I, P, I, P, P, P, I, P]
    lib.attn_fp8_prepare_ex.restype = I
    lib.attn_strerror.argtypes = [I]
    lib.attn_strerror.restype = ctypes.c_char_p
    _lib = lib
    return lib


def header_functions() -> list[str]:
    """Names of the functions include/attn.h declares."""
    text = open(HEADER).read()
    return re.findall(r"^(?:int|size_t|const char\*)\s+(attn_\w+)\s*\(", text, flags=re.M)


def attn_strerror(status: int) -> str:
    return load_library().attn_strerror(int(status)).decode()


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream_handle(stream, device=None):
    if stream is None:
        stream = torch.cuda.current_stream(device)
    return ctypes.c_void_p(stream.cuda_stream)


def _one_device(named):
    """The device every given tensor lives on (the library launches on that device)."""
    dev = None
    for name, t in named:
        if t is None:
            continue
        if dev is None:
            dev = t.device
        elif t.device != dev:
            raise ValueError(f"{name} is on {t.device}, expected {dev}: all tensors must share one GPU")
    return dev


def _check_tensor(t, name):
    if not isinstance(t, torch.Tensor):
        raise TypeError(f"{name} must be a torch.Tensor")
    if not t.is_cuda:
        raise ValueError(f"{name} must live on the GPU")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous (strided views are not supported)")


_FP8_TYPES = tuple(x for x in (getattr(torch, "float8_e4m3fn", None), torch.uint8) if x is not None)


def _dtype_code(t: torch.Tensor) -> int:
    if t.dtype == torch.bfloat16:
        return ATTN_BF16
    if t.dtype == torch.float16:
        return ATTN_FP16
    if t.dtype in _FP8_TYPES:
        return ATTN_FP8_E4M3
    raise TypeError(f"unsupported input dtype {t.dtype}")


def _fwd_call(q, k, v, o, lse, cu_seqlens, max_seqlen, q_scale, k_scale, v_scale, alpha):
    """Check the attn_fwd tensors; return the device and the C arguments around the mode."""
    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse)):
        _check_tensor(t, name)
    if lse.dtype != torch.float32:
        raise TypeError("lse must be float32")
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, N, Hq, d]")
        B, N, Hq, d = q.shape
        Hkv = k.shape[2]
    else:
        _check_tensor(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        if q.dim() != 3 or max_seqlen is None:
            raise ValueError("varlen q must be [T, Hq, d] and max_seqlen must be given")
        B = cu_seqlens.numel() - 1
        N = int(max_seqlen)
        _, Hq, d = q.shape
        Hkv = k.shape[1]
    kv_shape = (B, N, Hkv, d) if cu_seqlens is None else (q.shape[0], Hkv, d)
    lse_shape = (B, Hq, N) if cu_seqlens is None else (Hq, q.shape[0])
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"k and v must be {kv_shape}, got {tuple(k.shape)} and {tuple(v.shape)}")
    if tuple(o.shape) != tuple(q.shape) or tuple(lse.shape) != lse_shape:
        raise ValueError(f"o must be {tuple(q.shape)} and lse {lse_shape}")
    dt = _dtype_code(q)
    if _dtype_code(k) != dt or _dtype_code(v) != dt:
        raise TypeError("q, k and v must share one dtype")
    if dt != ATTN_FP8_E4M3:
        q_scale = k_scale = v_scale = None
    else:
        nblk = -(-N // 64)
        for name, t, H in (("q_scale", q_scale, Hq), ("k_scale", k_scale, Hkv), ("v_scale", v_scale, Hkv)):
            if t is not None:
                _check_tensor(t, name)
                if t.dtype != torch.float32 or tuple(t.shape) != (B, H, nblk):
                    raise ValueError(f"{name} must be float32 {(B, H, nblk)}")
        if o.dtype != torch.bfloat16:
            raise TypeError("o must be bfloat16 for fp8 inputs")
    if dt == ATTN_FP16 and o.dtype != torch.float16 or dt == ATTN_BF16 and o.dtype != torch.bfloat16:
        raise TypeError("o must have the dtype of q (bf16 or fp16)")
    alpha = (1.0 / d ** 0.5) if alpha is None else float(alpha)
    dev = _one_device((("q", q), ("k", k), ("v", v), ("o", o), ("lse", lse), ("cu_seqlens", cu_seqlens),
                       ("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)))
    head = (_ptr(q), _ptr(k), _ptr(v), _ptr(o), _ptr(lse), B, Hq, Hkv, N, _ptr(cu_seqlens), d)
    tail = (alpha, dt, _ptr(q_scale), _ptr(k_scale), _ptr(v_scale))
    return dev, head, tail


def attn_fwd(q, k, v, o, lse, *, causal: bool = False, alpha: float | None = None, cu_seqlens=None,
             max_seqlen: int | None = None, q_scale=None, k_scale=None, v_scale=None, stream=None) -> None:
    """Enqueue attn_fwd on ``stream`` (default: torch's current stream).

    Dense: q/o [B, N, Hq, d], k/v [B, N, Hkv, d], lse [B, Hq, N].
    Varlen: q/o [T, Hq, d], k/v [T, Hkv, d], lse [Hq, T], cu_seqlens int32 [B+1] on the GPU and
    ``max_seqlen`` >= the longest sequence.  fp8 inputs (float8_e4m3fn or uint8 codes) need the
    three per-block scale tensors.
    """
    dev, head, tail = _fwd_call(q, k, v, o, lse, cu_seqlens, max_seqlen, q_scale, k_scale, v_scale, alpha)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.attn_fwd(*head, int(bool(causal)), *tail, _stream_handle(stream, dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd")


def attn_fwd_window(q, k, v, o, lse, *, window: int, alpha: float | None = None, cu_seqlens=None,
                    max_seqlen: int | None = None, q_scale=None, k_scale=None, v_scale=None, stream=None) -> None:
    """Enqueue attn_fwd_window: causal attention in which query i sees keys i-window+1 .. i.
    Tensors as for :func:`attn_fwd`."""
    dev, head, tail = _fwd_call(q, k, v, o, lse, cu_seqlens, max_seqlen, q_scale, k_scale, v_scale, alpha)
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.attn_fwd_window(*head, int(window), *tail, _stream_handle(stream, dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fwd_window")


def check_cu_seqlens(cu_seqlens, total_tokens: int, max_seqlen: int | None = None) -> None:
    """Validate packed-layout offsets on the host before a call.  The library reads them on the
    device only and cannot check them; offsets that decrease or pass the tensors' tokens make
    its kernels access memory outside the tensors.  This copies them to the host, so it waits
    for the work that writes them: meant for debugging and input pipelines, not for every call.
    Raises ValueError unless cu_seqlens is a 1-D int32 tensor of at least two entries that
    starts at 0, never decreases and ends at ``total_tokens`` (the token count of q, k and v),
    and, when ``max_seqlen`` is given, no sequence is longer than it."""
    if not isinstance(cu_seqlens, torch.Tensor) or cu_seqlens.dim() != 1 or cu_seqlens.dtype != torch.int32:
        raise ValueError("cu_seqlens must be a 1-D int32 tensor")
    cu = cu_seqlens.cpu().tolist()
    if len(cu) < 2:
        raise ValueError("cu_seqlens needs at least two entries (one sequence)")
    if cu[0] != 0:
        raise ValueError(f"cu_seqlens[0] must be 0, got {cu[0]}")
    lengths = [b - a for a, b in zip(cu, cu[1:])]
    if min(lengths) < 0:
        raise ValueError(f"cu_seqlens decreases after entry {lengths.index(min(lengths))}")
    if cu[-1] != int(total_tokens):
        raise ValueError(f"cu_seqlens ends at {cu[-1]}, but the tensors hold {int(total_tokens)} tokens")
    if max_seqlen is not None and max(lengths) > int(max_seqlen):
        raise ValueError(f"a sequence of {max(lengths)} tokens is longer than max_seqlen = {int(max_seqlen)}")


def attention(q, k, v, *, causal: bool = False, alpha: float | None = None, cu_seqlens=None,
              max_seqlen: int | None = None, q_scale=None, k_scale=None, v_scale=None, window: int | None = None,
              stream=None):
    """Allocate O (bf16, or fp16 for fp16 inputs) and LSE (fp32) and call :func:`attn_fwd`, or,
    with ``window``, :func:`attn_fwd_window` (causal sliding window; ``causal`` is then implied).
    The outputs are allocated on ``stream`` (default: the current stream), the stream the
    kernel writes them on, so torch's caching allocator orders their reuse behind it."""
    with torch.cuda.stream(stream):
        out_dtype = torch.float16 if q.dtype == torch.float16 else torch.bfloat16
        o = torch.empty(q.shape, dtype=out_dtype, device=q.device)
        if cu_seqlens is None:
            B, N, Hq, _ = q.shape
            lse = torch.empty((B, Hq, N), dtype=torch.float32, device=q.device)
        else:
            T, Hq, _ = q.shape
            lse = torch.empty((Hq, T), dtype=torch.float32, device=q.device)
        kw = dict(alpha=alpha, cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, q_scale=q_scale, k_scale=k_scale,
                  v_scale=v_scale, stream=stream)
        if window is not None:
            attn_fwd_window(q, k, v, o, lse, window=window, **kw)
        else:
            attn_fwd(q, k, v, o, lse, causal=causal, **kw)
    return o, lse


def attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, workspace, *, causal: bool = False, alpha: float | None = None,
             cu_seqlens=None, max_seqlen: int | None = None, window: int | None = None, stream=None) -> None:
    """Enqueue attn_bwd: dq, dk, dv (q's, k's, v's layouts and dtype) of the attn_fwd call that
    produced o and lse, for the output gradient dout.  ``workspace``: float32 on the GPU with at
    least B * Hq * N elements (it receives D = rowsum(dout * o)).  With ``window``,
    attn_bwd_window (the causal sliding window of attn_fwd_window)."""
    dev, head, tail = _fwd_call(q, k, v, o, lse, cu_seqlens, max_seqlen, None, None, None, alpha)
    for name, t, ref in (("dout", dout, o), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(t, name)
        if t.dtype != ref.dtype or tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} must match {tuple(ref.shape)} {ref.dtype}")
    _check_tensor(workspace, "workspace")
    B, Hq, N = head[5], head[6], head[8]
    if workspace.dtype != torch.float32 or workspace.numel() < B * Hq * N:
        raise ValueError(f"workspace must be float32 with at least {B * Hq * N} elements")
    _one_device((("q", q), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv), ("workspace", workspace)))
    lib = load_library()
    alpha_v, dt = tail[0], tail[1]
    with torch.cuda.device(dev):
        args = (head[0], head[1], head[2], head[3], head[4], _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv),
                _ptr(workspace), B, Hq, head[7], N, head[9], head[10])
        if window is not None:
            st = lib.attn_bwd_window(*args, int(window), alpha_v, dt, _stream_handle(stream, dev))
        else:
            st = lib.attn_bwd(*args, int(bool(causal)), alpha_v, dt, _stream_handle(stream, dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_window" if window is not None else "attn_bwd")


def attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, *, causal: bool = False, alpha: float | None = None,
                     cu_seqlens=None, max_seqlen: int | None = None, stream=None) -> None:
    """Enqueue attn_bwd_noalloc: :func:`attn_bwd` without a workspace argument, for callers that
    cannot allocate (D lives in the library's static per-GPU array of ATTN_BWD_NOALLOC_MAX_ROWS
    floats; calls that overlap on one GPU race on it)."""
    dev, head, tail = _fwd_call(q, k, v, o, lse, cu_seqlens, max_seqlen, None, None, None, alpha)
    for name, t, ref in (("dout", dout, o), ("dq", dq, q), ("dk", dk, k), ("dv", dv, v)):
        _check_tensor(t, name)
        if t.dtype != ref.dtype or tuple(t.shape) != tuple(ref.shape):
            raise ValueError(f"{name} must match {tuple(ref.shape)} {ref.dtype}")
    _one_device((("q", q), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)))
    lib = load_library()
    B, Hq, N = head[5], head[6], head[8]
    with torch.cuda.device(dev):
        st = lib.attn_bwd_noalloc(head[0], head[1], head[2], head[3], head[4], _ptr(dout), _ptr(dq), _ptr(dk),
                                  _ptr(dv), B, Hq, head[7], N, head[9], head[10], int(bool(causal)), tail[0],
                                  tail[1], _stream_handle(stream, dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_bwd_noalloc")


def attention_backward(q, k, v, o, lse, dout, *, causal: bool = False, alpha: float | None = None, cu_seqlens=None,
                       max_seqlen: int | None = None, window: int | None = None, stream=None):
    """Allocate dq, dk, dv and the workspace and call :func:`attn_bwd`.  Everything is allocated
    on ``stream`` (default: the current stream), where the kernels run: the workspace is freed
    on return while they may still be running, and the allocator then hands its memory only to
    later work on that stream."""
    with torch.cuda.stream(stream):
        dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
        if cu_seqlens is None:
            B, N, Hq = q.shape[0], q.shape[1], q.shape[2]
        else:
            B, N, Hq = cu_seqlens.numel() - 1, int(max_seqlen), q.shape[1]
        ws = torch.empty(B * Hq * N, dtype=torch.float32, device=q.device)
        attn_bwd(q, k, v, o, lse, dout, dq, dk, dv, ws, causal=causal, alpha=alpha, cu_seqlens=cu_seqlens,
                 max_seqlen=max_seqlen, window=window, stream=stream)
    return dq, dk, dv


def _prepare_call(q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, hadamard_signs, cu_seqlens, max_seqlen, name):
    """Check the pre-pass tensors; return the device and (B, Hq, Hkv, N, d)."""
    for nm, t in (("q", q), ("k", k), ("v", v), ("q8", q8), ("k8", k8), ("v8", v8),
                  ("q_scale", q_scale), ("k_scale", k_scale), ("v_scale", v_scale)):
        _check_tensor(t, nm)
    if hadamard_signs is not None:
        _check_tensor(hadamard_signs, "hadamard_signs")
        if hadamard_signs.dtype != torch.int8:
            raise TypeError("hadamard_signs must be int8")
    if q.dtype != torch.bfloat16 or k.dtype != torch.bfloat16 or v.dtype != torch.bfloat16:
        raise TypeError(f"{name} takes bf16 inputs")
    if cu_seqlens is None:
        if q.dim() != 4:
            raise ValueError("dense q must be [B, N, Hq, d]")
        B, N, Hq, d = q.shape
        Hkv = k.shape[2]
        kv_shape = (B, N, Hkv, d)
    else:
        _check_tensor(cu_seqlens, "cu_seqlens")
        if cu_seqlens.dtype != torch.int32:
            raise TypeError("cu_seqlens must be int32")
        if q.dim() != 3 or max_seqlen is None:
            raise ValueError("packed q must be [T, Hq, d] and max_seqlen must be given")
        B, N = cu_seqlens.numel() - 1, int(max_seqlen)
        T, Hq, d = q.shape
        Hkv = k.shape[1]
        kv_shape = (T, Hkv, d)
    nblk = -(-N // 64)
    if tuple(k.shape) != kv_shape or tuple(v.shape) != kv_shape:
        raise ValueError(f"k and v must be {kv_shape}")
    for t, ref in ((q8, q), (k8, k), (v8, v)):
        if tuple(t.shape) != tuple(ref.shape) or t.element_size() != 1:
            raise ValueError("fp8 outputs must be 1-byte tensors shaped like their inputs")
    for t, H in ((q_scale, Hq), (k_scale, Hkv), (v_scale, Hkv)):
        if t.dtype != torch.float32 or tuple(t.shape) != (B, H, nblk):
            raise ValueError(f"scales must be float32 {(B, H, nblk)}")
    if hadamard_signs is not None and hadamard_signs.numel() != d:
        raise ValueError("hadamard_signs must have d entries")
    dev = _one_device((("q", q), ("k", k), ("v", v), ("q8", q8), ("k8", k8), ("v8", v8), ("q_scale", q_scale),
                       ("k_scale", k_scale), ("v_scale", v_scale), ("hadamard_signs", hadamard_signs),
                       ("cu_seqlens", cu_seqlens)))
    return dev, (B, Hq, Hkv, N, d)


def attn_fp8_prepare(q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, *, hadamard_signs=None,
                     stream=None) -> None:
    """Enqueue the FP8 pre-pass: bf16 q/k/v [B, N, H, d] -> e4m3 codes + fp32 block scales
    [B, H, ceil(N/64)].  ``hadamard_signs``: int8 [d] of +-1 on the GPU, or None for no rotation."""
    dev, (B, Hq, Hkv, N, d) = _prepare_call(q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, hadamard_signs,
                                            None, None, "attn_fp8_prepare")
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.attn_fp8_prepare(_ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale),
                                  _ptr(k_scale), _ptr(v_scale), B, Hq, Hkv, N, d, _ptr(hadamard_signs),
                                  _stream_handle(stream, dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_prepare")


def attn_fp8_prepare_ex(q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, *, scaling: int = ATTN_FP8_SCALE_BLOCK,
                        cu_seqlens=None, max_seqlen: int | None = None, rope_cos=None, rope_sin=None,
                        hadamard_signs=None, stream=None) -> None:
    """:func:`attn_fp8_prepare` for the dense or the packed layout (``cu_seqlens`` int32 [B+1]
    on the GPU, q [T, Hq, d], k/v [T, Hkv, d], ``max_seqlen`` >= the longest sequence; scales
    [B, H, ceil(max_seqlen/64)]), with ``scaling`` = ATTN_FP8_SCALE_BLOCK (one scale per
    64-token block) or ATTN_FP8_SCALE_TENSOR (one scale per tensor, in every block entry), and
    optionally fused with a rotary embedding (``rope_cos``, ``rope_sin``: float32 [P, d/2] with
    P >= the sequence length, position = token index within its sequence)."""
    dev, (B, Hq, Hkv, N, d) = _prepare_call(q, k, v, q8, k8, v8, q_scale, k_scale, v_scale, hadamard_signs,
                                            cu_seqlens, max_seqlen, "attn_fp8_prepare_ex")
    if (rope_cos is None) != (rope_sin is None):
        raise ValueError("rope_cos and rope_sin come together")
    if rope_cos is not None:
        for nm, t in (("rope_cos", rope_cos), ("rope_sin", rope_sin)):
            _check_tensor(t, nm)
            if t.dtype != torch.float32 or t.dim() != 2 or t.shape[1] != d // 2 or t.shape[0] < N:
                raise ValueError(f"{nm} must be float32 [P >= {N}, {d // 2}]")
        _one_device((("q", q), ("rope_cos", rope_cos), ("rope_sin", rope_sin)))
    lib = load_library()
    with torch.cuda.device(dev):
        st = lib.attn_fp8_prepare_ex(_ptr(q), _ptr(k), _ptr(v), _ptr(q8), _ptr(k8), _ptr(v8), _ptr(q_scale),
                                     _ptr(k_scale), _ptr(v_scale), B, Hq, Hkv, N, _ptr(cu_seqlens), d,
                                     _ptr(rope_cos), _ptr(rope_sin), _ptr(hadamard_signs), int(scaling),
                                     _stream_handle(stream, dev))
    if st != ATTN_OK:
        raise AttnError(st, "attn_fp8_prepare_ex")


def fp8_prepare(q, k, v, *, hadamard_signs=None, per_tensor: bool = False, cu_seqlens=None,
                max_seqlen: int | None = None, rope_cos=None, rope_sin=None, stream=None):
    """Allocate the e4m3 tensors (as uint8 codes) and scales and run the pre-pass, with one scale
    per 64-token block (:func:`attn_fp8_prepare`) or, with ``per_tensor``, one per tensor;
    ``cu_seqlens`` / ``max_seqlen`` select the packed layout (:func:`attn_fp8_prepare_ex`).
    The outputs are allocated on ``stream`` (default: the current stream), where the pre-pass
    writes them."""
    with torch.cuda.stream(stream):
        return _fp8_prepare_alloc(q, k, v, hadamard_signs, per_tensor, cu_seqlens, max_seqlen, rope_cos, rope_sin,
                                  stream)


def _fp8_prepare_alloc(q, k, v, hadamard_signs, per_tensor, cu_seqlens, max_seqlen, rope_cos, rope_sin, stream):
    if cu_seqlens is None:
        B, N, Hq, d = q.shape
        Hkv = k.shape[2]
    else:
        B, N = cu_seqlens.numel() - 1, int(max_seqlen)
        Hq, Hkv = q.shape[1], k.shape[1]
    nblk = -(-N // 64)
    dev = q.device
    q8 = torch.empty(q.shape, dtype=torch.uint8, device=dev)
    k8 = torch.empty(k.shape, dtype=torch.uint8, device=dev)
    v8 = torch.empty(v.shape, dtype=torch.uint8, device=dev)
    qs = torch.empty((B, Hq, nblk), dtype=torch.float32, device=dev)
    ks = torch.empty((B, Hkv, nblk), dtype=torch.float32, device=dev)
    vs = torch.empty((B, Hkv, nblk), dtype=torch.float32, device=dev)
    if per_tensor or cu_seqlens is not None or rope_cos is not None:
        attn_fp8_prepare_ex(q, k, v, q8, k8, v8, qs, ks, vs,
                            scaling=ATTN_FP8_SCALE_TENSOR if per_tensor else ATTN_FP8_SCALE_BLOCK,
                            cu_seqlens=cu_seqlens, max_seqlen=max_seqlen, rope_cos=rope_cos, rope_sin=rope_sin,
                            hadamard_signs=hadamard_signs, stream=stream)
    else:
        attn_fp8_prepare(q, k, v, q8, k8, v8, qs, ks, vs, hadamard_signs=hadamard_signs, stream=stream)
    return q8, k8, v8, qs, ks, vs
