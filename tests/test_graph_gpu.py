"""GPU: the entry points recorded into HIP graphs (torch.cuda.CUDAGraph), as a serving loop would
use them.  attn_fwd allocates nothing and attn_bwd_noalloc keeps its workspace in a static device
array, so each can be captured once and replayed.  Every graph is replayed three times; before each
replay new inputs are copied into the captured tensors and the outputs are overwritten with NaN
(eager work between replays), and after it the outputs must equal, bit for bit, an eager call on
the same inputs (the same kernels run either way).  Covered: the persistent short-sequence path,
a causal d = 64 and a causal d = 256 problem, packed sequences, and the allocation-free backward."""
import numpy as np
import pytest
import torch

import seeded_inputs as si
from tests import gpu_util as gu

FWD_CASES = [
    dict(B=2, N=600, Hq=4, Hkv=2, d=128, causal=False, varlen=None),  # persistent workgroups
    dict(B=2, N=333, Hq=4, Hkv=4, d=64, causal=True, varlen=None),
    dict(B=1, N=1100, Hq=2, Hkv=1, d=256, causal=True, varlen=None),
    dict(B=None, N=None, Hq=4, Hkv=2, d=128, causal=True, varlen=[300, 0, 77, 512]),
]


def _inputs(case, seed):
    if case["varlen"] is not None:
        return si.varlen_inputs(case["varlen"], case["Hq"], case["Hkv"], case["d"], causal=case["causal"], seed=seed)
    return si.dense_inputs(case["B"], case["N"], case["Hq"], case["d"], Hkv=case["Hkv"], causal=case["causal"],
                           seed=seed)


def _fwd(ea, q, k, v, o, lse, inp, cu):
    ea.attn_fwd(q, k, v, o, lse, causal=inp.causal, alpha=inp.alpha, cu_seqlens=cu,
                max_seqlen=inp.N if cu is not None else None)


@pytest.mark.gpu
@pytest.mark.parametrize("ci", range(len(FWD_CASES)))
def test_forward_graph_replays(ci):
    import exact_attention_76_amd as ea

    case = FWD_CASES[ci]
    inp = _inputs(case, 700 + 10 * ci)
    gu.say("graph forward", case)
    q, k, v, cu = gu.to_device(inp)
    o = torch.empty_like(q)
    lse_shape = (inp.B, inp.Hq, inp.N) if cu is None else (inp.Hq, q.shape[0])
    lse = torch.empty(lse_shape, dtype=torch.float32, device="cuda")
    _fwd(ea, q, k, v, o, lse, inp, cu)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        _fwd(ea, q, k, v, o, lse, inp, cu)
    torch.cuda.synchronize()
    for r in range(3):
        new = _inputs(case, 701 + 10 * ci + r)
        qn, kn, vn, _ = gu.to_device(new)
        q.copy_(qn)
        k.copy_(kn)
        v.copy_(vn)
        o.fill_(float("nan"))
        lse.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        o_ref, lse_ref = torch.empty_like(o), torch.empty_like(lse)
        _fwd(ea, qn, kn, vn, o_ref, lse_ref, new, cu)
        torch.cuda.synchronize()
        assert torch.equal(o, o_ref), f"replay {r}: O differs"
        assert torch.equal(lse, lse_ref), f"replay {r}: L differs"
        assert bool(torch.isfinite(o).all()) and bool(torch.isfinite(lse).all()), "rows left unwritten"


@pytest.mark.gpu
def test_noalloc_backward_graph_replays():
    import exact_attention_76_amd as ea

    inp = si.dense_inputs(2, 400, 4, 128, Hkv=2, causal=True, seed=790)
    gu.say("graph backward", inp.B, inp.N, inp.Hq, inp.Hkv, inp.d)
    q, k, v, _ = gu.to_device(inp)
    o, lse = ea.attention(q, k, v, causal=True, alpha=inp.alpha)
    dt = gu.torch_dtype(inp.dtype)
    as_dev = lambda bits: torch.from_numpy(bits.view(np.int16)).view(dt).cuda()
    dout = as_dev(si.output_gradient(inp, 791))
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ea.attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=True, alpha=inp.alpha)  # warm-up
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        ea.attn_bwd_noalloc(q, k, v, o, lse, dout, dq, dk, dv, causal=True, alpha=inp.alpha)
    torch.cuda.synchronize()
    for r in range(3):
        dout.copy_(as_dev(si.output_gradient(inp, 792 + r)))
        for t in (dq, dk, dv):
            t.fill_(float("nan"))
        g.replay()
        torch.cuda.synchronize()
        ref = ea.attention_backward(q, k, v, o, lse, dout, causal=True, alpha=inp.alpha)
        torch.cuda.synchronize()
        for name, got, want in zip(("dq", "dk", "dv"), (dq, dk, dv), ref):
            assert torch.equal(got, want), f"replay {r}: {name} differs"
