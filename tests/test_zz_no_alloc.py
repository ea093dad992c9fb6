"""attn_bwd_noalloc (the backward entry point for callers that cannot allocate) against attn_bwd
with a caller workspace, through the C ABI: the same kernels, so the gradients must be
bit-identical.  Two calls in a row on one GPU, the second with a smaller problem (the static
workspace keeps the first call's contents), plus packed sequences."""
import ctypes

import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _both(inp, seed):
    import exact_attention_76_amd as ea

    q, k, v, cu = gu.to_device(inp)
    N = inp.N
    kw = dict(causal=inp.causal, alpha=inp.alpha, cu_seqlens=cu, max_seqlen=N if cu is not None else None)
    o, lse = gu.attention_nan(q, k, v, **kw)
    do = torch.from_numpy(si.output_gradient(inp, seed).view(np.int16)).view(gu.torch_dtype(inp.dtype)).cuda()
    ref = ea.attention_backward(q, k, v, o, lse, do, **kw)
    got = tuple(torch.full_like(t, float("nan")) for t in (q, k, v))
    ea.attn_bwd_noalloc(q, k, v, o, lse, do, *got, **kw)
    torch.cuda.synchronize()
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g, r), f"{name}: attn_bwd_noalloc differs from attn_bwd"
        assert torch.isfinite(g).all()


def test_noalloc_matches_attn_bwd_twice_then_smaller():
    big = si.dense_inputs(2, 700, 8, 128, Hkv=2, causal=True, seed=900)
    small = si.dense_inputs(1, 130, 4, 64, Hkv=4, causal=False, seed=901)
    gu.say("noalloc backward: large then small")
    _both(big, 902)
    _both(small, 903)


def test_noalloc_packed():
    inp = si.varlen_inputs([0, 70, 300, 1, 129], 4, 2, 128, causal=True, seed=904)
    gu.say("noalloc backward: packed")
    _both(inp, 905)


def test_noalloc_rejects_oversize_without_launching():
    import exact_attention_76_amd as ea

    lib = ea.load_library()
    a = ctypes.c_void_p(1 << 20)  # a 16-byte aligned stand-in address; never dereferenced
    N = ea.ATTN_BWD_NOALLOC_MAX_ROWS // 16 + 1  # B = 1, Hq = 16: one row over
    st = lib.attn_bwd_noalloc(a, a, a, a, a, a, a, a, a, 1, 16, 16, N, None, 64, 0, 0.125, ea.ATTN_BF16, None)
    assert st == ea.ATTN_ERR_TOO_LARGE
    assert "static workspace" in ea.attn_strerror(st)
