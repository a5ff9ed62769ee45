"""Pins of the rotary embedding oracle and of BlockAttention with it (CPU).

* the d = 4 closed form, element by element (tests/golden/rope_cases.json):
  pins the rotate-half pairing and the frequencies;
* position 0 is the identity, norms are kept, the inverse undoes it;
* q.k after rotation depends only on the difference of the positions;
* block attention gives the same result with positions counted from each
  block's first token as from the sequence's (the reason the kernels count
  from the block start);
* central finite differences of the gradients through the rotation;
* planted mistakes (interleaved pairing, wrong sign, wrong frequencies, the
  backward's rotation left out) are rejected.
"""

import importlib
import json
import math
import os

import numpy as np
import pytest

import oracle
rope_mod = importlib.import_module("oracle.rope")   # the module (the package exports its function as oracle.rope)
from jagged_attention_ads_amd.workloads import offsets_from_lengths

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden", "rope_cases.json")


def _closed_form(x, p, base):
    a0, a1 = p, p * base ** -0.5
    return [x[0] * math.cos(a0) - x[2] * math.sin(a0), x[1] * math.cos(a1) - x[3] * math.sin(a1),
            x[2] * math.cos(a0) + x[0] * math.sin(a0), x[3] * math.cos(a1) + x[1] * math.sin(a1)]


def _check_closed_form(rope_fn):
    for c in json.load(open(GOLDEN))["cases"]:
        x = np.array(c["x"], dtype=np.float64).reshape(1, 1, 4)
        got = rope_fn(x, [c["position"]], c["base"])[0, 0]
        if not np.allclose(got, _closed_form(c["x"], c["position"], c["base"]), rtol=0, atol=1e-14):
            return False
    return True


def test_closed_form():
    assert _check_closed_form(oracle.rope)


def test_identity_norm_inverse():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((50, 3, 64))
    pos = rng.integers(0, 5000, 50)
    assert np.array_equal(oracle.rope(x[:1], [0]), x[:1])
    y = oracle.rope(x, pos)
    # every (i, i + d/2) pair keeps its length
    h = 32
    assert np.allclose(y[..., :h] ** 2 + y[..., h:] ** 2, x[..., :h] ** 2 + x[..., h:] ** 2, rtol=0, atol=1e-12)
    assert np.allclose(oracle.rope(y, pos, inverse=True), x, rtol=0, atol=1e-12)


def _relative(rope_fn):
    rng = np.random.default_rng(2)
    q, k = rng.standard_normal((1, 1, 128)), rng.standard_normal((1, 1, 128))
    for m, n, sh in [(5, 2, 100), (0, 63, 7), (1000, 3, 33)]:
        a = float(np.sum(rope_fn(q, [m]) * rope_fn(k, [n])))
        b = float(np.sum(rope_fn(q, [m + sh]) * rope_fn(k, [n + sh])))
        if abs(a - b) > 1e-9:
            return False
    return True


def test_scores_depend_on_position_difference_only():
    assert _relative(oracle.rope)


def test_block_positions_equal_sequence_positions():
    rng = np.random.default_rng(3)
    lengths = [130, 64, 1, 65, 200]
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    q, k, v = (rng.standard_normal((T, 2, 32)) for _ in range(3))
    s = 1.0 / math.sqrt(32)
    for act, causal in [("softmax", True), ("softmax", False), ("silu", True)]:
        out, lse = oracle.attention_fwd(q, k, v, off, off, s, act, causal, block=64, rope_base=10000.0)
        # positions from each 64-token block's first token instead
        bpos = oracle.sequence_positions(off) % 64
        qb, kb = oracle.rope(q, bpos), oracle.rope(k, bpos)
        out2, lse2 = oracle.attention_fwd(qb, kb, v, off, off, s, act, causal, block=64)
        assert np.allclose(out, out2, rtol=0, atol=1e-12)
        if lse is not None:
            assert np.allclose(lse, lse2, rtol=0, atol=1e-12)


@pytest.mark.parametrize("act,causal", [("softmax", True), ("softmax", False), ("silu", True)])
def test_finite_differences(act, causal):
    rng = np.random.default_rng(4)
    lengths = [5, 3, 7]
    off = offsets_from_lengths(lengths)
    T, H, d = int(off[-1]), 1, 6
    q, k, v, do = (rng.standard_normal((T, H, d)) for _ in range(4))
    s = 0.7
    dq, dk, dv = oracle.attention_bwd(q, k, v, do, off, off, s, act, causal, block=4, rope_base=50.0)

    def loss(qq, kk, vv):
        o, _ = oracle.attention_fwd(qq, kk, vv, off, off, s, act, causal, block=4, rope_base=50.0)
        return float(np.sum(o * do))
    eps = 1e-6
    for name, x, g in (("q", q, dq), ("k", k, dk), ("v", v, dv)):
        num = np.zeros_like(x)
        for idx in np.ndindex(x.shape):
            xp, xm = x.copy(), x.copy()
            xp[idx] += eps
            xm[idx] -= eps
            args_p = {"q": (xp, k, v), "k": (q, xp, v), "v": (q, k, xp)}[name]
            args_m = {"q": (xm, k, v), "k": (q, xm, v), "v": (q, k, xm)}[name]
            num[idx] = (loss(*args_p) - loss(*args_m)) / (2 * eps)
        assert np.allclose(g, num, rtol=1e-6, atol=1e-7), name


# ---------------------------------------------------------------- planted mistakes

def _interleaved(x, positions, base=10000.0, inverse=False):
    x = np.asarray(x, dtype=np.float64)
    ang = rope_mod.rope_angles(positions, x.shape[-1], base)[:, None, :]
    s = -np.sin(ang) if inverse else np.sin(ang)
    a, b = x[..., 0::2], x[..., 1::2]
    out = np.empty_like(x)
    out[..., 0::2], out[..., 1::2] = a * np.cos(ang) - b * s, b * np.cos(ang) + a * s
    return out


def _wrong_sign(x, positions, base=10000.0, inverse=False):
    return oracle.rope(x, positions, base, inverse=not inverse)


def _wrong_freq(x, positions, base=10000.0, inverse=False):
    return oracle.rope(x, positions, base ** 0.5, inverse)


def test_mutants_are_rejected():
    for m in (_interleaved, _wrong_sign, _wrong_freq):
        assert not _check_closed_form(m), m.__name__
    # the backward without turning the gradients back: finite differences disagree
    rng = np.random.default_rng(5)
    off = offsets_from_lengths([6])
    q, k, v, do = (rng.standard_normal((6, 1, 4)) for _ in range(4))
    dq_r, _, _ = oracle.attention_bwd(*rope_mod_inputs(q, k, off), v, do, off, off, 1.0, "softmax", True)
    dq, _, _ = oracle.attention_bwd(q, k, v, do, off, off, 1.0, "softmax", True, rope_base=10000.0)
    assert not np.allclose(dq_r, dq, rtol=0, atol=1e-6)


def rope_mod_inputs(q, k, off):
    pos = oracle.sequence_positions(off)
    return oracle.rope(q, pos), oracle.rope(k, pos)
