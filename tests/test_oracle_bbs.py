"""Pins of the Base Batch Shuffling oracle (CPU only).

* worked examples derived by hand (tests/golden/bbs_cases.json);
* brute force: for an even number of base batches, merging the k-th
  heaviest with the k-th lightest gives the smallest possible largest merged
  load over every way of pairing them (the exchange argument: pairing a
  heavier with a lighter never raises the larger of two sums);
* invariants: the plan is a permutation of the samples, every merged batch
  is whole base batches, loads are conserved;
* planted mistakes in copies of the oracle are rejected by these pins.
"""

import itertools
import json
import os

import numpy as np
import pytest

import oracle
from oracle import bbs

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "bbs_cases.json")


def _cases():
    with open(GOLDEN) as f:
        return json.load(f)["cases"]


@pytest.mark.parametrize("case", _cases(), ids=lambda c: c["name"])
def test_worked_examples(case):
    perm, start = oracle.bbs_plan(case["lengths"], case["base_batch"], case["cost"])
    assert perm == case["perm"]
    assert start == case["batch_start"]
    assert oracle.merged_loads(case["lengths"], perm, start, case["cost"]) == case["loads"]


def _pairings(items):
    """Every way of splitting an even-sized list into unordered pairs."""
    if not items:
        yield []
        return
    a = items[0]
    for i in range(1, len(items)):
        rest = items[1:i] + items[i + 1:]
        for p in _pairings(rest):
            yield [(a, items[i])] + p


def _min_max_pair_load(loads):
    return min(max(loads[a] + loads[b] for a, b in p) for p in _pairings(list(range(len(loads)))))


def _check_optimal(plan_fn):
    rng = np.random.default_rng(11)
    for trial in range(60):
        nb = 2 * int(rng.integers(1, 5))                # 2 .. 8 base batches
        base = int(rng.integers(1, 4))
        lengths = [int(x) for x in rng.integers(0, 50, nb * base)]
        cost = "tokens" if trial % 2 else "pairs"
        perm, start = plan_fn(lengths, base, cost)
        loads = [sum(bbs.sample_cost(lengths[i], cost) for i in range(s, e)) for s, e in bbs.base_batches(len(lengths), base)]
        got = max(oracle.merged_loads(lengths, perm, start, cost))
        if got != _min_max_pair_load(loads):
            return False
    return True


def test_pairing_minimises_the_largest_merged_load():
    assert _check_optimal(oracle.bbs_plan)


def _check_invariants(plan_fn):
    rng = np.random.default_rng(12)
    for _ in range(40):
        n = int(rng.integers(0, 40))
        base = int(rng.integers(1, 6))
        lengths = [int(x) for x in rng.integers(0, 300, n)]
        perm, start = plan_fn(lengths, base, "tokens")
        if sorted(perm) != list(range(n)) or start[0] != 0 or start[-1] != n:
            return False
        bases = {tuple(range(s, e)) for s, e in bbs.base_batches(n, base)}
        for i in range(len(start) - 1):
            seg = perm[start[i]:start[i + 1]]
            # whole base batches, in input order within each
            parts, k = [], 0
            while k < len(seg):
                for b in bases:
                    if seg[k:k + len(b)] == list(b):
                        parts.append(b)
                        k += len(b)
                        break
                else:
                    return False
            if not 1 <= len(parts) <= 2:
                return False
        if sum(oracle.merged_loads(lengths, perm, start)) != sum(lengths):
            return False
    return True


def test_invariants():
    assert _check_invariants(oracle.bbs_plan)


# ---------------------------------------------------------------- planted mistakes

def _mutant(pairing=None, descending=True):
    """A copy of the oracle's plan with one step changed."""
    def plan(lengths, base_batch=128, cost="tokens"):
        bases = bbs.base_batches(len(lengths), base_batch)
        loads = [sum(bbs.sample_cost(lengths[i], cost) for i in range(s, e)) for s, e in bases]
        order = sorted(range(len(bases)), key=lambda k: ((-loads[k]) if descending else loads[k], k))
        n = len(order)
        groups = pairing(order) if pairing else [[order[i], order[n - 1 - i]] for i in range(n // 2)]
        if n % 2 and not pairing:
            groups.append([order[n // 2]])
        perm, start = [], [0]
        for grp in groups:
            for k in grp:
                perm.extend(range(*bases[k]))
            start.append(len(perm))
        return perm, start
    return plan


def test_mutants_are_rejected():
    # heaviest with the next heaviest (adjacent pairs) instead of the lightest
    adjacent = _mutant(pairing=lambda o: [o[i:i + 2] for i in range(0, len(o), 2)])
    assert not _check_optimal(adjacent)
    # lightest first: the same pairs in the opposite order, caught by the worked examples
    asc = _mutant(descending=False)
    c = _cases()[0]
    assert asc(c["lengths"], c["base_batch"], c["cost"]) != (c["perm"], c["batch_start"])
    # the median base batch dropped for an odd count
    drop = _mutant(pairing=lambda o: [[o[i], o[len(o) - 1 - i]] for i in range(len(o) // 2)])
    assert not _check_invariants(drop)
