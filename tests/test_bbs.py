"""The library's Base Batch Shuffling (host C++, through the C ABI) against
the oracle's, bit for bit (integer work), and its argument checks.  CPU only:
the batch former runs on the host."""

import numpy as np
import pytest

import oracle
from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import WORKLOADS, draw_lengths


@pytest.mark.parametrize("cost", ["tokens", "pairs"])
@pytest.mark.parametrize("n,base", [(0, 128), (1, 128), (127, 128), (256, 128), (1024, 128), (1000, 128),
                                    (9, 2), (37, 5), (3000, 7)])
def test_matches_oracle(n, base, cost):
    rng = np.random.default_rng(n * 31 + base)
    lengths = rng.integers(0, 2048, n).astype(np.int32)
    perm, start = jfa.jfa_bbs_plan(lengths, base, cost)
    ref_perm, ref_start = oracle.bbs_plan(lengths.tolist(), base, cost)
    assert perm.tolist() == ref_perm
    assert start.tolist() == ref_start


@pytest.mark.parametrize("name", ["selfattn_causal", "pareto_train"])
def test_workload_lengths(name):
    """The benchmark's length laws, 8 steps of base batches."""
    wl = WORKLOADS[name]
    lengths = draw_lengths(np.random.default_rng(5), wl.q_law, 128 * 16).astype(np.int32)
    for cost in ("tokens", "pairs"):
        perm, start = jfa.jfa_bbs_plan(lengths, 128, cost)
        ref_perm, ref_start = oracle.bbs_plan(lengths.tolist(), 128, cost)
        assert perm.tolist() == ref_perm and start.tolist() == ref_start


def test_rejects():
    L = jfa.lib()
    perm = np.empty(4, np.int64)
    start = np.empty(4, np.int64)
    lens = np.array([1, 2, 3, 4], np.int32)
    assert L.jfa_bbs_plan(lens.ctypes.data, -1, 2, 0, perm.ctypes.data, start.ctypes.data) == 1
    assert L.jfa_bbs_plan(lens.ctypes.data, 4, 0, 0, perm.ctypes.data, start.ctypes.data) == 1
    assert L.jfa_bbs_plan(lens.ctypes.data, 4, 2, 2, perm.ctypes.data, start.ctypes.data) == 1
    assert L.jfa_bbs_plan(None, 4, 2, 0, perm.ctypes.data, start.ctypes.data) == 1
    bad = np.array([1, -2, 3, 4], np.int32)
    assert L.jfa_bbs_plan(bad.ctypes.data, 4, 2, 0, perm.ctypes.data, start.ctypes.data) == 1
    assert L.jfa_bbs_batch_count(4, 2) == 1 and L.jfa_bbs_batch_count(5, 2) == 2
    assert L.jfa_bbs_batch_count(0, 2) == 0 and L.jfa_bbs_batch_count(4, 0) == 0
