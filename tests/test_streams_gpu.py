"""GPU tests of stream ordering in the Python binding: every call enqueues on the stream it is
given (default: torch's current stream) and never synchronises, so work queued earlier on that
stream must finish first, and tensors the allocating helpers create or free belong to that
stream.  Each case puts slow matrix products ahead of the call on a side stream, so a launch
on the wrong stream would read its inputs before they are written, and a workspace handed back
to the current stream too early would be overwritten while the kernels still read it.  The
results must equal those of the same calls made without any side stream, bit for bit (the
same kernels on the same inputs)."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests import gpu_util as gu


def _slow_work():
    """About ten milliseconds of matrix products on the current stream."""
    x = torch.randn(4096, 4096, device="cuda")
    for _ in range(8):
        x = (x @ x) * (1.0 / 4096)
    return x


def _inputs(causal=False, seed=41):
    return gu.to_device(si.dense_inputs(2, 1024, 8, 128, Hkv=2, causal=causal, seed=seed))


@pytest.mark.gpu
@pytest.mark.parametrize("how", ["current", "argument"])
def test_forward_waits_for_its_stream(how):
    import exact_attention_76_amd as ea

    q, k, v, _ = _inputs()
    o_ref, lse_ref = ea.attention(q, k, v)
    torch.cuda.synchronize()
    gu.say("forward on a side stream", how)
    s = torch.cuda.Stream()
    q2 = torch.zeros_like(q)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        _slow_work()
        q2.copy_(q)  # ready only after the slow work
    if how == "current":
        with torch.cuda.stream(s):
            o, lse = ea.attention(q2, k, v)
    else:
        o, lse = ea.attention(q2, k, v, stream=s)
    torch.cuda.synchronize()
    assert torch.equal(o, o_ref) and torch.equal(lse, lse_ref)


@pytest.mark.gpu
@pytest.mark.parametrize("causal", [False, True])
def test_backward_workspace_stays_with_its_stream(causal):
    """attention_backward frees its workspace when it returns, while its kernels are still
    queued behind the slow work; allocations of the same size on the current stream, filled at
    once, must not receive that memory."""
    import exact_attention_76_amd as ea

    q, k, v, _ = _inputs(causal, seed=42)
    o, lse = ea.attention(q, k, v, causal=causal)
    do = torch.randn_like(q)
    ref = ea.attention_backward(q, k, v, o, lse, do, causal=causal)
    torch.cuda.synchronize()
    ws_numel = q.shape[0] * q.shape[2] * q.shape[1]
    gu.say("backward on a side stream", causal)
    s = torch.cuda.Stream()
    s.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(s):
        _slow_work()
    got = ea.attention_backward(q, k, v, o, lse, do, causal=causal, stream=s)
    junk = [torch.full((ws_numel,), float("nan"), device="cuda") for _ in range(4)]
    torch.cuda.synchronize()
    del junk
    for name, g, r in zip(("dq", "dk", "dv"), got, ref):
        assert torch.equal(g, r), name


@pytest.mark.gpu
def test_fp8_prepare_on_a_side_stream():
    import exact_attention_76_amd as ea

    q, k, v, _ = _inputs(seed=43)
    sg = torch.from_numpy(si.hadamard_signs(128, seed=55)).cuda()
    ref = ea.fp8_prepare(q, k, v, hadamard_signs=sg)
    torch.cuda.synchronize()
    gu.say("fp8 pre-pass on a side stream")
    s = torch.cuda.Stream()
    k2 = torch.zeros_like(k)
    torch.cuda.synchronize()
    with torch.cuda.stream(s):
        _slow_work()
        k2.copy_(k)
    got = ea.fp8_prepare(q, k2, v, hadamard_signs=sg, stream=s)
    torch.cuda.synchronize()
    for g, r in zip(got, ref):
        assert torch.equal(g, r)
    assert np.isfinite(got[4].cpu().numpy()).all()
