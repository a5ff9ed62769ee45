"""Host-side accounting of bench.py, checked by brute force over the
oracle's visibility mask: the useful-FLOP pair count and the number of
32 x 32 dS blocks that hold a visible pair (the blocks the dK/dV pass
stores and the dQ pass reads, which set their algorithmic bytes)."""

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
    from jagged_attention_ads_amd.workloads import WORKLOADS
    wl = WORKLOADS["selfattn_causal"]
    acct = bench.kernel_accounting(wl, 1000, 1000, 12345, 77, True)
    H, d = wl.heads, wl.head_dim
    assert acct["fwd"]["flops"] == 4 * d * H * 12345
    assert acct["bwd_dkdv"]["flops"] == 8 * d * H * 12345
    assert acct["bwd_dq"]["flops"] == 2 * d * H * 12345
    # the dS store: 77 blocks of 32 x 32 bf16 per head, written by dK/dV and read by dQ
    ds = 77 * H * 32 * 32 * 2
    no_ds = bench.kernel_accounting(wl, 1000, 1000, 12345, 77, False)
    assert acct["bwd_dkdv"]["bytes"] - no_ds["bwd_dkdv"]["bytes"] == ds
    assert acct["bwd_dq"]["bytes"] >= ds
