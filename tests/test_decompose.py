"""The work decomposition (exact_attention_76_amd/csrc/decompose.h) on the CPU, on the grids the
kernels launch.  decompose() maps a hardware workgroup id to the (query block, head, sequence)
it computes; the header is compiled for the host with a small harness (tests/decompose_host.cpp).

* It must be a bijection onto every (query block, head, sequence) of the grid: a block no
  workgroup computes would leave rows of O unwritten, a block computed twice would waste a
  workgroup (and race).  Checked for the five workloads' grids (16-bit forward: 256 queries per
  workgroup; FP8: 128; backward dQ: 128 queries, dK/dV: 256 keys per KV head) and for the head
  counts that take each branch (whole KV groups per XCD, single query heads per XCD, and the
  contiguous-range fallback when Hq is not a multiple of 8).
* Dispatch is round-robin over the 8 XCDs (id mod 8).  When Hq is a multiple of 8 every XCD must
  receive exactly the same work -- counted as visible (query, key) pairs, so packed sequences of
  unequal length and causal blocks of unequal size are weighed as they run -- and a KV group's
  query heads must stay on one XCD (they share its K/V in that XCD's L2).
* Causal grids start each XCD's longest blocks first (query block index non-increasing in
  dispatch order; in the fallback, within each (sequence, head) of the XCD's range).
"""
from __future__ import annotations

import os
import shutil
import subprocess

import numpy as np
import pytest

import seeded_inputs as si

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
CSRC = os.path.join(ROOT, "exact_attention_76_amd", "csrc")
HIPCC = os.environ.get("HIPCC", "/opt/rocm/bin/hipcc")
XCDS = 8

pytestmark = pytest.mark.skipif(shutil.which(HIPCC) is None and not os.path.exists(HIPCC),
                                reason="hipcc not available")


@pytest.fixture(scope="module")
def harness(tmp_path_factory):
    exe = str(tmp_path_factory.mktemp("decompose") / "decompose_host")
    subprocess.run([HIPCC, "--offload-arch=gfx950", "-O1", "-std=c++17", "-I", CSRC,
                    os.path.join(ROOT, "tests", "decompose_host.cpp"), "-o", exe], check=True,
                   capture_output=True)
    return exe


def mapping(exe, nqb, Hq, Hkv, B, causal):
    out = subprocess.run([exe, str(nqb), str(Hq), str(Hkv), str(B), str(int(causal))], check=True,
                         capture_output=True).stdout
    return np.frombuffer(out, dtype=np.int32).reshape(-1, 3)


def block_work(qb, lengths, br, causal):
    """Visible (query, key) pairs of each (query block, sequence) entry."""
    n = lengths[qb[:, 1]]
    q0 = qb[:, 0].astype(np.int64) * br
    rows = np.clip(n - q0, 0, br)
    if not causal:
        return rows * n
    # queries q0 .. q0 + rows - 1 see q0 + 1 .. q0 + rows keys
    return rows * q0 + rows * (rows + 1) // 2


def check_grid(exe, lengths, Hq, Hkv, br, causal, *, balanced):
    lengths = np.asarray(lengths, dtype=np.int64)
    B = len(lengths)
    nqb = -(-int(lengths.max()) // br)
    m = mapping(exe, nqb, Hq, Hkv, B, causal)
    qb, h, b = m[:, 0], m[:, 1], m[:, 2]
    assert m.shape[0] == nqb * Hq * B
    assert qb.min() >= 0 and qb.max() < nqb and h.min() >= 0 and h.max() < Hq and b.min() >= 0 and b.max() < B
    ids = (b.astype(np.int64) * Hq + h) * nqb + qb
    assert np.array_equal(np.sort(ids), np.arange(nqb * Hq * B)), "not a bijection"
    xcd = np.arange(len(m)) % XCDS
    if balanced:
        work = block_work(np.stack([qb, b], 1), lengths, br, causal)
        per_xcd = np.bincount(xcd, weights=work, minlength=XCDS)
        assert per_xcd.min() == per_xcd.max(), f"per-XCD work differs: {per_xcd}"
        group = h // (Hq // Hkv)
        if Hkv % XCDS == 0:  # a KV group's query heads stay on one XCD
            for g in np.unique(group):
                assert len(np.unique(xcd[group == g])) == 1, f"KV group {g} spans XCDs"
    if causal:
        for x in range(XCDS):
            sel = xcd == x
            if Hq % XCDS == 0:  # all of an XCD's blocks, longest first
                assert np.all(np.diff(qb[sel]) <= 0), f"XCD {x}: causal blocks not longest first"
            else:  # contiguous ranges: each (sequence, head) longest first
                for key in np.unique(b[sel] * Hq + h[sel]):
                    run = qb[sel][(b[sel] * Hq + h[sel]) == key]
                    assert np.all(np.diff(run) <= 0), f"XCD {x}: causal blocks not longest first"
    return m


def c4_lengths():
    return si.varlen_lengths(np.random.default_rng(4), 8, 256, 8192)


# (name, sequence lengths, Hq, Hkv, queries per workgroup, causal)
WORKLOAD_GRIDS = (
    [(f"C2 N={N} bf16", [N] * (16384 // N), 16, 16, 256, False) for N in (512, 1024, 2048, 4096, 8192, 16384)]
    + [("C1 bf16", [128], 2, 2, 256, False),
       ("C3 bf16 causal", [8192] * 2, 16, 16, 256, True),
       ("C4 bf16 packed causal GQA", None, 32, 8, 256, True),
       ("C5 fp8", [8192] * 2, 16, 16, 128, False),
       ("C3 fp8 causal", [8192] * 2, 16, 16, 128, True),
       ("C4 fp8 packed causal GQA", None, 32, 8, 128, True),
       ("C2 N=16384 backward dQ", [16384], 16, 16, 128, False),
       ("C3 backward dQ", [8192] * 2, 16, 16, 128, True),
       ("C4 backward dQ", None, 32, 8, 128, True),
       ("C2 N=16384 backward dK/dV", [16384], 16, 16, 256, False),
       ("C3 backward dK/dV", [8192] * 2, 16, 16, 256, True),
       ("C4 backward dK/dV (grid over KV heads)", None, 8, 8, 256, True)])


@pytest.mark.parametrize("name,lengths,Hq,Hkv,br,causal", WORKLOAD_GRIDS, ids=[g[0] for g in WORKLOAD_GRIDS])
def test_workload_grids(harness, name, lengths, Hq, Hkv, br, causal):
    lengths = c4_lengths() if lengths is None else lengths
    check_grid(harness, lengths, Hq, Hkv, br, causal, balanced=Hq % XCDS == 0)


# head splits of every branch: KV groups of 1 and 3 heads on one XCD, one query head at a time
# (Hkv not a multiple of 8), and the contiguous-range fallback (Hq not a multiple of 8)
SPLITS = [(8, 8), (24, 8), (16, 4), (8, 1), (8, 2), (12, 4), (2, 2), (6, 3), (40, 8), (64, 16),
          (1, 1), (3, 1), (5, 5), (7, 1), (10, 2), (14, 7)]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("Hq,Hkv", SPLITS)
def test_head_splits(harness, Hq, Hkv, causal):
    for lengths in ([300] * 3, [1], [700, 33, 256, 1, 513], [0, 5, 0, 130, 0]):
        lengths = np.maximum(np.asarray(lengths), 0)
        if lengths.max() == 0:
            continue
        check_grid(harness, lengths, Hq, Hkv, 256, causal, balanced=False)
        check_grid(harness, lengths, Hq, Hkv, 128, causal, balanced=False)


def test_balance_is_checked():
    """The balance check itself fails on a plainly unbalanced assignment (contiguous ranges of
    (sequence, head, block) ids per XCD on the packed workload, the previous decomposition)."""
    lengths = c4_lengths()
    nqb, Hq, B = -(-int(lengths.max()) // 256), 32, len(lengths)
    total = nqb * Hq * B
    logical = np.arange(total)
    per = total // XCDS
    xcd = logical // per
    qb, bh = logical % nqb, logical // nqb
    work = block_work(np.stack([qb, bh // Hq], 1), lengths, 256, True)
    per_xcd = np.bincount(xcd, weights=work, minlength=XCDS)
    assert per_xcd.max() / per_xcd.min() > 1.2
