"""GPU parity at the largest size the boundary accepts.

attn_fwd addresses one head's K/V rows with 32-bit byte offsets and accepts N * Hkv * d * 2 up to
2^31 - 1 bytes (larger calls return ATTN_ERR_UNSUPPORTED, checked on the CPU in test_abi).  Here
every head dim runs causal attention with N = 131071 and Hkv chosen so that a head's K/V rows
span just under 2 GiB: the last tiles sit at the top of the offset range.  The inputs (2.1 GB per
tensor) come from a seeded generator on the device; the oracle gets the K/V columns of the
sampled heads only and checks sampled rows, among them the first and the last tokens.
"""
import numpy as np
import pytest
import torch

import oracle
from tests import gpu_util as gu

pytestmark = pytest.mark.gpu

N = 131071


def _bits_to_f64(t: torch.Tensor) -> np.ndarray:
    return oracle.bf16_to_f64(t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16))


@pytest.mark.parametrize("d,H", [(64, 128), (128, 64), (256, 32)])
def test_largest_kv_span(d, H):
    import exact_attention_76_amd as ea

    span = (N - 1) * H * d * 2 + d * 2
    assert N * H * d * 2 <= 2**31 - 1 and span > 2**31 - 2**24  # just under the limit
    gu.say("largest K/V span", f"N={N} H={H} d={d} span={span}")
    gen = torch.Generator(device="cuda")
    gen.manual_seed(900 + d)
    q, k, v = (torch.randn((1, N, H, d), generator=gen, device="cuda", dtype=torch.float32).to(torch.bfloat16)
               for _ in range(3))
    alpha = d ** -0.5
    o, lse = ea.attention(q, k, v, causal=True, alpha=alpha)
    torch.cuda.synchronize()
    assert bool(torch.isfinite(lse).all()), "non-finite LSE"

    heads = np.array([0, H // 2, H - 1])
    rng = np.random.default_rng(d)
    tokens = np.concatenate([np.array([0, 1, 63, N // 2, N - 65, N - 2, N - 1]), rng.integers(0, N, 9)])
    # the oracle sees the selected heads only, renumbered 0.., each with its own K/V head
    qs, ks, vs = (_bits_to_f64(t[:, :, heads, :]) for t in (q, k, v))
    rows_h = np.repeat(np.arange(len(heads)), len(tokens))
    rows_t = np.tile(tokens, len(heads))
    o_ref, lse_ref = oracle.attention_rows(qs, ks, vs, rows_h, rows_t, causal=True, alpha=alpha)
    o_got = o[0, rows_t, heads[rows_h]].double().cpu().numpy()
    lse_got = lse[0, heads[rows_h], rows_t].double().cpu().numpy()
    m = gu.metrics(o_got, o_ref, lse_got, lse_ref, "bf16")
    gu.say("largest K/V span", m)
    gu.check(m, what=f"N={N} H={H} d={d}")
    del q, k, v, o, lse
    torch.cuda.empty_cache()
