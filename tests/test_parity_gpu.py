"""GPU parity of attn_fwd (16-bit inputs) against the fp64 oracle on the same seeded inputs.

* small problems that span several 256-query and 64-key tiles with ragged tails, on both
  sides of every loop-shape switch: every element of O and LSE is compared;
* closed forms the kernel must reproduce: a causal first row is a bit-exact copy of V_0;
  Q = 0 gives the mean of the visible V rows and L = ln(count);
* the five workloads at full size, in the benchmark's launch configuration: O and LSE start as
  NaN and must come back finite everywhere (every row written), every O element inside the
  range of its V column; the oracle checks one row of every (sequence, head, query block),
  i.e. of every workgroup, and two whole heads on every element.

Tolerances (bf16 bars; fp16 uses the same): O max-abs <= 1e-2 beyond the half ulp that
rounding the exact result to the output format costs by itself, O RMSE <= 2e-3, LSE max-abs
<= 1e-3.
"""
import numpy as np
import pytest
import torch

import oracle
import seeded_inputs as si
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu


def _compare_full(inp, what):
    gu.say(what, f"B={inp.B} N={inp.N} Hq={inp.Hq} Hkv={inp.Hkv} d={inp.d} causal={inp.causal} "
                 f"dtype={inp.dtype} seed={inp.seed} cu={None if inp.cu_seqlens is None else inp.cu_seqlens.tolist()}")
    o_gpu, lse_gpu = gu.run_gpu(inp)
    o_ref, lse_ref = gu.oracle_full(inp)
    m = gu.metrics(o_gpu, o_ref, lse_gpu, lse_ref, inp.dtype)
    gu.check(m, what=what)
    return m


def test_smallest_workload_every_element():
    _compare_full(si.CONFIGS["mha_b1_h2_n128_d64"](), "B1 H2 N128 d64")


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
def test_ragged_multi_tile(d, causal, dtype):
    inp = si.dense_inputs(2, 300, 4, d, Hkv=2, causal=causal, seed=100 + d + 7 * causal, dtype=dtype)
    _compare_full(inp, f"ragged d={d} causal={causal} {dtype}")


# Non-causal d = 128 takes the plain tile loop up to 512 keys per sequence and the ping-pong
# loop above that: both sides of the switch, with ragged query blocks and key tiles.
@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
@pytest.mark.parametrize("N", [512, 513, 700])
def test_noncausal_d128_both_loops(N, dtype):
    inp = si.dense_inputs(2, N, 4, 128, Hkv=2, causal=False, seed=900 + N, dtype=dtype)
    _compare_full(inp, f"non-causal d=128 N={N} {dtype}")


@pytest.mark.parametrize("lengths", [[300, 512, 5], [700, 33, 513, 1]])
def test_varlen_noncausal_d128_both_loops(lengths):
    inp = si.varlen_inputs(lengths, 4, 2, 128, causal=False, seed=910 + len(lengths))
    _compare_full(inp, f"varlen non-causal d=128 lengths={lengths}")


# Dense non-causal d = 128 with at most 1024 keys and an even number of 64-key tiles runs
# persistent workgroups (one per CU, each taking every G-th query block in turn).  B is chosen so
# that there are more blocks than CUs (several blocks per workgroup, the last workgroups one
# fewer), or fewer (one block each); odd tile counts (N = 576) take the per-block loops.  Hq = 12
# (not a multiple of the 8 XCDs) takes the decomposition's contiguous-range branch.
@pytest.mark.parametrize("N,B,Hq,Hkv,dtype", [(512, 32, 16, 16, "bf16"), (640, 5, 24, 8, "fp16"), (1000, 3, 32, 8, "bf16"),
                                              (1024, 2, 16, 4, "bf16"), (128, 1, 4, 2, "bf16"), (576, 4, 8, 8, "bf16"),
                                              (512, 16, 12, 4, "bf16")])
def test_persistent_blocks(N, B, Hq, Hkv, dtype):
    inp = si.dense_inputs(B, N, Hq, 128, Hkv=Hkv, causal=False, seed=930 + N, dtype=dtype)
    _compare_full(inp, f"persistent blocks N={N} B={B} Hq={Hq} Hkv={Hkv} {dtype}")


@pytest.mark.parametrize("N", [512, 1024])
def test_persistent_and_per_block_loops_bit_identical(N):
    """The persistent stream takes each block's tiles in the same order with the same arithmetic
    as the per-block loops, so the same data given as equal packed sequences (which take the
    plain loop at 512 keys and the ping-pong loop at 1024) must give the same bits."""
    import torch

    B, H = 6, 16
    inp = si.dense_inputs(B, N, H, 128, causal=False, seed=940 + N)
    gu.say("persistent vs per-block loops", N)
    q, k, v, _ = gu.to_device(inp)
    o1, l1 = gu.attention_nan(q, k, v, causal=False, alpha=inp.alpha)
    cu = torch.arange(0, (B + 1) * N, N, dtype=torch.int32, device="cuda")
    flat = [t.reshape(B * N, H, 128) for t in (q, k, v)]
    o2, l2 = gu.attention_nan(*flat, causal=False, alpha=inp.alpha, cu_seqlens=cu, max_seqlen=N)
    torch.cuda.synchronize()
    o1, l1 = o1.float().cpu().numpy().reshape(B * N, H, 128), l1.cpu().numpy()
    o2, l2 = o2.float().cpu().numpy(), l2.cpu().numpy()
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
    assert np.array_equal(o1, o2)
    # LSE: dense [B, H, N], packed [H, T]
    assert np.array_equal(l1.transpose(1, 0, 2).reshape(H, B * N), l2)


@pytest.mark.parametrize("dtype", ["bf16", "fp16"])
def test_plain_and_ping_pong_loops_bit_identical(dtype):
    """Both tile loops take the same tiles in the same key order with the same arithmetic, so
    they must agree bit for bit.  The same packed non-causal d = 128 inputs run the plain loop
    with max_seqlen = 512 and the ping-pong loop with max_seqlen = 1000 (a larger bound only
    grows the grid; the extra blocks exit)."""
    import torch

    inp = si.varlen_inputs([300, 5, 512, 129], 4, 2, 128, causal=False, seed=920, dtype=dtype)
    gu.say("plain vs ping-pong loop", dtype)
    q, k, v, cu = gu.to_device(inp)
    outs = []
    for max_seqlen in (512, 1000):
        o, lse = gu.attention_nan(q, k, v, causal=False, alpha=inp.alpha, cu_seqlens=cu, max_seqlen=max_seqlen)
        torch.cuda.synchronize()
        outs.append((o.float().cpu().numpy(), lse.cpu().numpy()))
    (o1, l1), (o2, l2) = outs
    assert np.all(np.isfinite(o1)) and np.all(np.isfinite(l1))
    assert np.array_equal(o1, o2) and np.array_equal(l1, l2)
    _compare_full(inp, f"plain loop, packed non-causal {dtype}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_varlen_small(d, causal):
    inp = si.varlen_inputs([1, 77, 300, 129, 64, 128], 4, 1, d, causal=causal, seed=200 + d)
    _compare_full(inp, f"varlen small d={d} causal={causal}")


# Head counts that take each branch of the work decomposition: heads spread over the 8 XCDs in
# whole KV groups (Hkv a multiple of 8, groups of 1 and 3 query heads), one query head at a
# time (Hq a multiple of 8 only), or the contiguous-range fallback (Hq not a multiple of 8);
# odd batch, ragged multi-tile length, every element compared.
@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,d", [(8, 8, 128), (24, 8, 128), (16, 4, 128), (8, 1, 256), (8, 2, 64), (12, 4, 128)])
def test_head_splits_over_xcds(Hq, Hkv, d, causal):
    inp = si.dense_inputs(3, 300, Hq, d, Hkv=Hkv, causal=causal, seed=700 + Hq + 3 * Hkv + d + causal)
    _compare_full(inp, f"head split Hq={Hq} Hkv={Hkv} d={d} causal={causal}")


@pytest.mark.parametrize("Hq,Hkv", [(16, 4), (16, 8)])
def test_varlen_head_splits(Hq, Hkv):
    """Packed sequences of unequal length with the per-XCD head split (by head and by group)."""
    inp = si.varlen_inputs([700, 33, 256, 1, 513], Hq, Hkv, 128, causal=True, seed=800 + Hq + Hkv)
    _compare_full(inp, f"varlen head split Hq={Hq} Hkv={Hkv}")


ODD_HEADS = [(1, 1, 128), (3, 1, 64), (5, 5, 128), (7, 1, 256), (10, 2, 128), (14, 7, 64)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv,d", ODD_HEADS)
def test_odd_head_counts(Hq, Hkv, d, causal):
    """Head counts that do not split evenly over the eight XCDs: one head, primes, groups of
    five and seven query heads per KV head; dense and packed."""
    seed = 900 + Hq + 3 * Hkv + d + causal
    inp = si.dense_inputs(2, 333, Hq, d, Hkv=Hkv, causal=causal, seed=seed)
    _compare_full(inp, f"odd heads Hq={Hq} Hkv={Hkv} d={d} causal={causal}")
    inp = si.varlen_inputs([333, 0, 95, 512], Hq, Hkv, d, causal=causal, seed=seed + 1)
    _compare_full(inp, f"odd heads packed Hq={Hq} Hkv={Hkv} d={d} causal={causal}")


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128, 256])
@pytest.mark.parametrize("B,N", [(300, 1), (97, 3), (33, 65)])
def test_many_tiny_sequences(B, N, d, causal):
    """Large batches of sequences shorter than one tile (or one key past it): every block is a
    ragged tail."""
    inp = si.dense_inputs(B, N, 4, d, Hkv=2, causal=causal, seed=1000 + B + N + d + causal)
    _compare_full(inp, f"tiny sequences B={B} N={N} d={d} causal={causal}")


def test_varlen_max_seqlen_above_longest():
    """N larger than every sequence only grows the grid; extra blocks exit."""
    inp = si.varlen_inputs([5, 130], 2, 2, 128, causal=True, seed=300)
    inp.N = 1000
    _compare_full(inp, "varlen with slack max_seqlen")


@pytest.mark.parametrize("causal", [False, True])
def test_varlen_empty_sequences(causal):
    """Zero-length sequences anywhere in the pack (first, middle, last) write nothing and leave
    their neighbours' rows exact."""
    inp = si.varlen_inputs([0, 5, 0, 130, 0], 4, 2, 128, causal=causal, seed=302)
    _compare_full(inp, f"varlen with empty sequences causal={causal}")


def test_single_token_sequence():
    inp = si.dense_inputs(3, 1, 2, 128, causal=False, seed=301)
    _compare_full(inp, "N=1")


@pytest.mark.parametrize("d", [64, 128, 256])
def test_causal_first_row_is_exact_copy(d):
    inp = si.dense_inputs(2, 200, 4, d, Hkv=2, causal=True, seed=400 + d)
    gu.say("causal row 0 copy", d)
    o, lse = gu.run_gpu(inp)
    v = oracle.widen(inp.v, "bf16")
    for h in range(4):
        assert np.array_equal(o[:, 0, h], v[:, 0, h // 2]), "O_0 must equal V_0 bit for bit"
    q, k = oracle.widen(inp.q, "bf16"), oracle.widen(inp.k, "bf16")
    s00 = inp.alpha * np.einsum("bhd,bhd->bh", q[:, 0], np.repeat(k[:, 0], 2, axis=1))
    assert np.max(np.abs(lse[:, :, 0] - s00)) <= gu.TOL_LSE


@pytest.mark.parametrize("causal", [False, True])
def test_uniform_scores_give_mean(causal):
    inp = si.dense_inputs(1, 333, 2, 128, causal=causal, seed=500)
    inp.q[...] = 0  # +0.0 in bf16
    gu.say("uniform scores", causal)
    o, lse = gu.run_gpu(inp)
    v = oracle.widen(inp.v, "bf16")
    cnt = np.arange(1, 334, dtype=np.float64) if causal else np.full(333, 333.0)
    mean = (np.cumsum(v, axis=1) / cnt[None, :, None, None]) if causal else \
        np.repeat(v.mean(axis=1, keepdims=True), 333, axis=1)
    m = gu.metrics(o, mean, lse, np.log(cnt)[None, None, :].repeat(2, 1), "bf16")
    gu.check(m, what=f"uniform causal={causal}")


FULL = [n for n in si.CONFIGS if not n.startswith("fp8")]
BR16 = 256  # queries per workgroup of the 16-bit kernels


@pytest.mark.parametrize("name", FULL)
def test_full_size(name):
    """The workload at full size in the launch configuration the benchmark times.  O and LSE
    start as NaN, so finiteness everywhere proves every row was written; every element is a
    convex combination of its V column; the oracle checks one row of every (sequence, head,
    query block) -- every workgroup of the grid -- and two whole heads on every element."""
    inp = si.CONFIGS[name]()
    gu.say("full size", name, f"T={inp.total_tokens}")
    o_gpu, lse_gpu = gu.run_gpu(inp)
    assert np.all(np.isfinite(o_gpu)) and np.all(np.isfinite(lse_gpu)), "rows left unwritten"
    v = oracle.widen(inp.v, inp.dtype)
    vmax = float(np.max(np.abs(v)))
    assert float(np.max(np.abs(o_gpu))) <= vmax * (1 + 2 ** -7)
    heads, tokens = gu.coverage_rows(inp, BR16, seed=1)
    q, k, v = gu.widened(inp)
    o_ref, lse_ref = oracle.attention_rows(q, k, v, heads, tokens, causal=inp.causal, alpha=inp.alpha,
                                           cu_seqlens=inp.cu_seqlens)
    o_s, lse_s = gu.gpu_rows(inp, o_gpu, lse_gpu, heads, tokens)
    gu.say("full size rows checked", len(heads))
    gu.check(gu.metrics(o_s, o_ref, lse_s, lse_ref, inp.dtype), what=name)
