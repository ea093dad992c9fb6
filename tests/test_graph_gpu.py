"""GPU: the entry points recorded into HIP graphs (torch.cuda.CUDAGraph), as a serving loop would
use them.  attn_fwd allocates nothing and attn_bwd_noalloc keeps its workspace in a static device
array, so each can be captured once and replayed.  Every graph is replayed three times; before each
replay new inputs are copied into the captured tensors and the outputs are overwritten with NaN
(eager work between replays), and after it the outputs must equal, bit for bit, an eager call on
the same inputs (the same kernels run either way).  Covered: the persistent short-sequence path,
a causal d = 64 and a causal d = 256 problem, packed sequences, the allocation-free backward, and
the FP8 pipeline (pre-pass and attention in one graph) with block and per-tensor scales, with the
rotary embedding and on packed sequences."""
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


FP8_CASES = [
    dict(per_tensor=False, rope=False, varlen=None, causal=False),
    dict(per_tensor=True, rope=False, varlen=None, causal=True),   # three pre-pass kernels
    dict(per_tensor=False, rope=True, varlen=[300, 0, 200], causal=True),
]


def _fp8_inputs(case, seed):
    if case["varlen"] is not None:
        return si.varlen_inputs(case["varlen"], 8, 2, 128, causal=case["causal"], seed=seed)
    return si.dense_inputs(2, 320, 8, 128, Hkv=2, causal=case["causal"], seed=seed)


@pytest.mark.gpu
@pytest.mark.parametrize("ci", range(len(FP8_CASES)))
def test_fp8_pipeline_graph_replays(ci):
    """attn_fp8_prepare_ex (bf16 Q, K, V -> e4m3 codes and scales) followed by attn_fwd on the codes,
    recorded into one graph: every replay's codes, scales, O and L equal an eager run's."""
    import exact_attention_76_amd as ea

    case = FP8_CASES[ci]
    inp = _fp8_inputs(case, 810 + 10 * ci)
    gu.say("graph fp8 pipeline", case)
    q, k, v, cu = gu.to_device(inp)
    packed = {} if cu is None else dict(cu_seqlens=cu, max_seqlen=inp.N)
    sg = torch.from_numpy(si.hadamard_signs(128, seed=55)).cuda()
    rope = {}
    if case["rope"]:
        cos, sin = si.rope_tables(inp.N, 128)
        rope = dict(rope_cos=torch.from_numpy(cos).cuda(), rope_sin=torch.from_numpy(sin).cuda())
    scaling = ea.ATTN_FP8_SCALE_TENSOR if case["per_tensor"] else ea.ATTN_FP8_SCALE_BLOCK
    nblk = -(-inp.N // 64)
    lse_shape = (inp.B, inp.Hq, inp.N) if cu is None else (inp.Hq, q.shape[0])

    def buffers():
        return dict(q8=torch.empty(q.shape, dtype=torch.uint8, device="cuda"),
                    k8=torch.empty(k.shape, dtype=torch.uint8, device="cuda"),
                    v8=torch.empty(v.shape, dtype=torch.uint8, device="cuda"),
                    qs=torch.empty((inp.B, inp.Hq, nblk), dtype=torch.float32, device="cuda"),
                    ks=torch.empty((inp.B, inp.Hkv, nblk), dtype=torch.float32, device="cuda"),
                    vs=torch.empty((inp.B, inp.Hkv, nblk), dtype=torch.float32, device="cuda"),
                    o=torch.empty(q.shape, dtype=torch.bfloat16, device="cuda"),
                    lse=torch.empty(lse_shape, dtype=torch.float32, device="cuda"))

    def pipeline(qq, kk, vv, b):
        ea.attn_fp8_prepare_ex(qq, kk, vv, b["q8"], b["k8"], b["v8"], b["qs"], b["ks"], b["vs"], scaling=scaling,
                               hadamard_signs=sg, **packed, **rope)
        ea.attn_fwd(b["q8"], b["k8"], b["v8"], b["o"], b["lse"], causal=inp.causal, alpha=inp.alpha,
                    q_scale=b["qs"], k_scale=b["ks"], v_scale=b["vs"], **packed)

    bufs = buffers()
    pipeline(q, k, v, bufs)  # warm-up outside the capture
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        pipeline(q, k, v, bufs)
    torch.cuda.synchronize()
    for r in range(3):
        new = _fp8_inputs(case, 811 + 10 * ci + r)
        qn, kn, vn, _ = gu.to_device(new)
        q.copy_(qn)
        k.copy_(kn)
        v.copy_(vn)
        for t in bufs.values():
            t.fill_(float("nan") if t.dtype.is_floating_point else 0xAB)
        g.replay()
        torch.cuda.synchronize()
        ref = buffers()
        pipeline(qn, kn, vn, ref)
        torch.cuda.synchronize()
        for name in bufs:
            got, want = bufs[name], ref[name]
            if name in ("qs", "ks", "vs") and cu is not None:
                # packed: the scale entries past a sequence's last block are not written
                nb = -(-np.diff(inp.cu_seqlens) // 64)
                live = torch.from_numpy(np.arange(nblk)[None, :] < nb[:, None]).cuda()[:, None, :].expand_as(got)
                got, want = got[live], want[live]
            assert torch.equal(got, want), f"replay {r}: {name} differs"
        assert bool(torch.isfinite(bufs["o"]).all()) and bool(torch.isfinite(bufs["lse"]).all()), "rows left unwritten"
