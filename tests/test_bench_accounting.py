"""Host-side accounting of bench.py, checked by brute force over the
oracle's visibility mask: the useful-FLOP pair count and the number of
32 x 32 dS blocks that hold a visible pair (the blocks the dK/dV pass
stores and the dQ pass reads, reported as workspace traffic), and the
per-kernel algorithmic bytes: the method's own tensors, each once."""

import importlib.util
import os

import numpy as np
import pytest

import oracle

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
_spec = importlib.util.spec_from_file_location("bench", os.path.join(ROOT, "bench.py"))
bench = importlib.util.module_from_spec(_spec)
_spec.loader.exec_module(bench)


def _cases():
    rng = np.random.default_rng(3)
    yield [1, 31, 32, 33, 64, 100], [1, 31, 32, 33, 64, 100]
    yield [0, 5, 70, 3], [4, 0, 70, 200]
    yield list(rng.integers(0, 140, 12)), list(rng.integers(0, 140, 12))


@pytest.mark.parametrize("causal", [False, True])
def test_visible_pairs_and_ds_blocks(causal):
    for lq, lk in _cases():
        pairs = bench.visible_pairs(lq, lk, causal)
        blocks = 0
        for b, (q, k) in enumerate(zip(lq, lk)):
            vis = oracle.visible_mask(q, k, causal)
            assert pairs[b] == vis.sum()
            for i0 in range(0, q, 32):
                for j0 in range(0, k, 32):
                    blocks += bool(vis[i0:i0 + 32, j0:j0 + 32].any())
        assert bench.ds_blocks(lq, lk, causal) == blocks


def test_kernel_accounting_shapes():
    """Algorithmic bytes are the method's own tensors, each once; the dS
    blocks the library stores and reads back are workspace traffic, reported
    apart."""
    from jagged_attention_ads_amd.workloads import WORKLOADS
    wl = WORKLOADS["selfattn_causal"]
    acct = bench.kernel_accounting(wl, 1000, 900, 12345, 77, True)
    H, d, es = wl.heads, wl.head_dim, 2
    assert acct["fwd"]["flops"] == 4 * d * H * 12345
    assert acct["bwd_dkdv"]["flops"] == 8 * d * H * 12345
    assert acct["bwd_dq"]["flops"] == 2 * d * H * 12345
    q, k, row = 1000 * H * d * es, 900 * H * d * es, 1000 * H * 4
    assert acct["fwd"]["bytes"] == 2 * q + 2 * k + row                  # Q, K, V read; O, lse written
    assert acct["bwd_dkdv"]["bytes"] == 2 * q + 2 * k + 2 * row + 2 * k  # Q, dO, K, V, lse, delta; dK, dV
    assert acct["bwd_dq"]["bytes"] == k + q                              # K read, dQ written
    # the dS store: 77 blocks of 32 x 32 bf16 per head, not algorithmic
    ds = 77 * H * 32 * 32 * 2
    no_ds = bench.kernel_accounting(wl, 1000, 900, 12345, 77, False)
    assert acct["bwd_dkdv"]["bytes"] == no_ds["bwd_dkdv"]["bytes"]
    assert acct["bwd_dkdv"]["ds_store_bytes"] == ds and acct["bwd_dq"]["ds_store_bytes"] == ds
    assert no_ds["bwd_dkdv"]["ds_store_bytes"] == 0


@pytest.mark.parametrize("causal", [False, True])
def test_short_split(causal):
    """The short sequences (<= 64 queries, 1 .. 64 keys) whose dQ the dK/dV
    pass writes: their rows, pairs and dS blocks by brute force, and moving
    them out of the dQ pass leaves the backward's FLOPs at 10 d per pair over
    stored dS (the recomputing dQ pass adds S and dP again: 4 d per pair of
    the sequences it takes)."""
    from jagged_attention_ads_amd.workloads import WORKLOADS
    wl = WORKLOADS["selfattn_causal"]
    for lq, lk in _cases():
        sq = sk = sp = sb = 0
        for q, k in zip(lq, lk):
            if q <= 64 and 1 <= k <= 64:
                vis = oracle.visible_mask(q, k, causal)
                sq, sk, sp = sq + q, sk + k, sp + int(vis.sum())
                sb += sum(bool(vis[i0:i0 + 32, j0:j0 + 32].any()) for i0 in range(0, q, 32) for j0 in range(0, k, 32))
        short = bench.short_split(lq, lk, causal)
        assert short == (sq, sk, sp, sb)
        pairs = int(bench.visible_pairs(lq, lk, causal).sum())
        nb = bench.ds_blocks(lq, lk, causal)
        T_q, T_k = int(np.sum(lq)), int(np.sum(lk))
        for ds_path in (True, False):
            a = bench.kernel_accounting(wl, T_q, T_k, pairs, nb, ds_path, short)
            b = bench.kernel_accounting(wl, T_q, T_k, pairs, nb, ds_path)
            dH = wl.head_dim * wl.heads
            assert a["bwd_dkdv"]["flops"] + a["bwd_dq"]["flops"] == dH * (10 * pairs if ds_path else
                                                                           14 * pairs - 4 * sp)
            assert a["bwd_dq"]["bytes"] <= b["bwd_dq"]["bytes"]
