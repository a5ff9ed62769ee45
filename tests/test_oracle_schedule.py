"""Pins of the scheduler's CPU work-list enumeration (CPU only).

The tile costs are checked against brute force over every (query, key) pair of
every tile; the ordering against its definition as properties.
"""

import numpy as np
import pytest

import oracle
from jagged_attention_ads_amd.workloads import offsets_from_lengths


def _sees(i, j, lq, lk, causal):
    return 0 <= j < lk and 0 <= i < lq and (not causal or i - j >= lq - lk)


def _brute_fwd_cost(lq, lk, t, bm, bn, causal):
    last_block = -1
    for i in range(t * bm, min((t + 1) * bm, lq)):
        for j in range(lk):
            if _sees(i, j, lq, lk, causal):
                last_block = max(last_block, j // bn)
    return last_block + 1


def _brute_kv_cost(lq, lk, t, bm, bn, causal):
    blocks = set()
    for j in range(t * bn, min((t + 1) * bn, lk)):
        for i in range(lq):
            if _sees(i, j, lq, lk, causal):
                blocks.add(i // bm)
    if not blocks:
        return 0
    return -(-lq // bm) - min(blocks)


LENGTH_SETS = [
    ([1, 17, 64, 65, 130, 0, 3], [1, 17, 64, 65, 130, 0, 3]),
    ([5, 40, 0, 200, 64], [90, 3, 7, 0, 257]),
    ([128, 127, 129, 1000], [128, 127, 129, 1000]),
]


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("bm,bn", [(64, 64), (128, 64), (32, 64), (64, 32), (16, 128)])
@pytest.mark.parametrize("ls", range(len(LENGTH_SETS)))
def test_tile_costs_brute_force(ls, bm, bn, causal):
    lq, lk = LENGTH_SETS[ls]
    qo, ko = offsets_from_lengths(lq), offsets_from_lengths(lk)
    fwd = oracle.fwd_tile_costs(qo, ko, bm, bn, causal)
    kv = oracle.kv_tile_costs(qo, ko, bm, bn, causal)
    for b in range(len(lq)):
        assert [t for t, _ in fwd[b]] == list(range(-(-lq[b] // bm)))
        assert [t for t, _ in kv[b]] == list(range(-(-lk[b] // bn)))
        for t, c in fwd[b]:
            assert c == _brute_fwd_cost(lq[b], lk[b], t, bm, bn, causal), (b, t)
        for t, c in kv[b]:
            assert c == _brute_kv_cost(lq[b], lk[b], t, bm, bn, causal), (b, t)


@pytest.mark.parametrize("causal", [False, True])
def test_worklist_order(causal):
    rng = np.random.default_rng(3)
    lq = rng.integers(0, 300, size=40)
    lk = rng.integers(0, 300, size=40)
    qo, ko = offsets_from_lengths(lq), offsets_from_lengths(lk)
    H = 3
    costs = oracle.fwd_tile_costs(qo, ko, 64, 64, causal)
    items = oracle.worklist(costs, H)
    expected = {(b, h, t): c for b, tl in enumerate(costs) for h in range(H) for t, c in tl}
    assert len(items) == len(expected)
    assert {(b, h, t) for b, h, t, _ in items} == set(expected)
    for b, h, t, c in items:
        assert expected[(b, h, t)] == c
    for a, z in zip(items, items[1:]):
        assert a[3] >= z[3]
        if a[3] == z[3]:
            assert a[:3] < z[:3]
