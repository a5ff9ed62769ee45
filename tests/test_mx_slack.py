"""Pins of the MXFP8 allowances (tests.mx_util.fwd_slack, bwd_slack): the
oracle itself, run with the values it quantises perturbed within the stated
error, never moves its outputs by more than the allowance; and the
per-element allowance has its closed forms.  The allowances only take
error off the GPU gates, so what matters is that they cover what they
claim (brute force here) and stay small (the separation of plausible
mistakes, test_mx_bwd_gates_separate_mistakes, is checked with them)."""

import numpy as np
import pytest

import oracle.mx as mx
from tests.gpu_util import beyond_slack
from tests.mx_util import _flip_allowance, bwd_slack, fwd_slack, score_error


def _draw(lq, lk, heads, d, seed, causal):
    rng = np.random.default_rng(seed)
    qo = np.concatenate([[0], np.cumsum(lq)])
    ko = np.concatenate([[0], np.cumsum(lk)])
    q, k, v, do = (rng.standard_normal((n, heads, d)) for n in (qo[-1], ko[-1], ko[-1], qo[-1]))
    return q, k, v, do, qo, ko


# ------------------------------------------------------------------ per-element allowance

def test_flip_allowance_closed_forms():
    sc = 2.0 ** -3
    # one column, one block: max 48 (exponent -3: 48 in (28, 56], 384 scaled)
    x = np.zeros((32, 1))
    x[0] = 48.0
    x[1] = (1 + 1 / 16) * sc        # midpoint of 1 and 1.125 (scaled): one step either way
    x[2] = 1.25 * sc                # representable, 1/16 from both midpoints
    x[3] = 2.0 ** -12               # 2^-9 scaled: the smallest subnormal
    a = _flip_allowance(x, 1e-9, 0)
    assert a[1, 0] == 0.125 * sc
    assert a[2, 0] == 0.0 and a[3, 0] == 0.0 and a[0, 0] == 0.0
    assert not a[4:].any()
    # the block max at 448 2^-3: the exponent may become -2, under which
    # 2^-12 is 2^-10 and rounds to 0 (the tie goes to the even code)
    x[0] = 56.0
    a = _flip_allowance(x, 1e-9, 0)
    assert a[0, 0] == 0.0 and a[3, 0] == 2.0 ** -12
    assert a[1, 0] == 0.125 * sc   # 1.0625 2^-3 is 0.53125 2^-2: a midpoint there too
    # along rows: the same values transposed give the transposed allowance
    np.testing.assert_array_equal(_flip_allowance(x.T, 1e-9, 1), a.T)
    # no error, no allowance
    assert not _flip_allowance(np.random.default_rng(0).standard_normal((70, 9)), 0.0, 0).any()


@pytest.mark.parametrize("axis", [0, 1])
def test_flip_allowance_covers_perturbations(axis):
    """Brute force: x' anywhere within rel |x| of x (the interval ends, and
    random points) quantises within the allowance of Q(x), for blocks whose
    largest element sits at an exponent's bound and for random ones."""
    rng = np.random.default_rng(11 + axis)
    for trial in range(12):
        x = rng.standard_normal((70, 40)) * np.exp2(rng.integers(-20, 20, size=(1, 40)))
        x[rng.random(x.shape) < 0.1] = 0
        if trial % 2:   # largest magnitudes exactly at 448 2^k or 224 2^k
            for c in range(0, 40, 3):
                r = int(rng.integers(0, 32))
                x[r, c] = (448.0 if c % 2 else 224.0) * 2.0 ** int(rng.integers(-10, 5))
                x[:32, c] = np.clip(x[:32, c], -abs(x[r, c]), abs(x[r, c]))
        rel = 10.0 ** rng.uniform(-7, -1, size=x.shape)
        xx, rr = (x, rel) if axis == 0 else (x.T, rel.T)
        a = _flip_allowance(xx, rr, axis)
        ref = mx.mx_quantize_matrix(xx, axis)
        for _ in range(12):
            u = rng.choice([-1.0, 1.0, 0.0], size=xx.shape) * rng.random(xx.shape) ** 0.1
            d = np.abs(mx.mx_quantize_matrix(xx * (1 + u * rr), axis) - ref)
            assert np.all(d <= a), (trial, np.max(d - a))


def test_beyond_slack():
    r = np.array([1.0, 1.0, 1.0, -2.0])
    g = np.array([1.5, 0.7, 1.05, -2.0])
    np.testing.assert_allclose(beyond_slack(g, r, np.array([0.1, 0.1, 0.1, 0.1])), [1.4, 0.8, 1.0, -2.0])


# ------------------------------------------------------------------ forward and backward allowances

@pytest.mark.parametrize("causal", [False, True])
def test_fwd_slack_covers_perturbed_scores(causal, monkeypatch):
    """The oracle's forward with every score t (log2 units) moved within
    0.95 of score_error's bound before the weights are quantised -- a block
    floor or an E4M3 decision may go the other way -- stays within
    fwd_slack of the unperturbed output; and the allowance is a small part
    of the output."""
    q, k, v, _, qo, ko = _draw([1, 37, 70, 100], [40, 37, 70, 64], 2, 64, 5, causal)
    scale = 0.3
    ref, _ = mx.mx_attention_fwd(q, k, v, qo, ko, scale, causal)
    slack = fwd_slack(q, k, v, qo, ko, scale, causal)
    # the bound of every (sequence, head) block, in the oracle's order
    qh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(q))
    kh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(k))
    c = scale / np.log(2.0)
    bounds = [score_error(qh[qo[b]:qo[b + 1], h], kh[ko[b]:ko[b + 1], h],
                          c * (qh[qo[b]:qo[b + 1], h] @ kh[ko[b]:ko[b + 1], h].T), c)
              for b in range(len(qo) - 1) if qo[b + 1] > qo[b] and ko[b + 1] > ko[b] for h in range(q.shape[1])]
    rng = np.random.default_rng(6)
    orig = mx.quantize_p
    moved = 0.0
    for trial in range(6):
        calls = iter(bounds)
        amp = 0.95 * (1.0 if trial % 2 else rng.random())
        monkeypatch.setattr(mx, "quantize_p",
                            lambda t, vis: orig(t + amp * next(calls) * rng.uniform(-1, 1, t.shape), vis))
        got, _ = mx.mx_attention_fwd(q, k, v, qo, ko, scale, causal)
        d = np.abs(got - ref)
        assert np.all(d <= slack + 1e-12), np.max(d - slack)
        moved = max(moved, d.max())
    assert moved > 0   # the perturbations do flip decisions
    assert np.linalg.norm(slack) < 0.05 * np.linalg.norm(ref)


def test_fwd_slack_floor_flip_closed_form():
    """One query, 32 keys: the largest score 3 + 1e-4 (log2 units), within
    the bound of the integer 3, so the block's floor may be 2 -- the largest
    weight then saturates at 448 2^-6 = 7 instead of 2^8 2^-5 = 8 (the
    E4M3 value of 2^(3 + 1e-4)), 1/8 of it less."""
    d = 32
    q = np.zeros((1, 1, d))
    k = np.zeros((32, 1, d))
    v = np.zeros((32, 1, d))
    q[0, 0, 0] = 1.0
    k[:, 0, 0] = -4.0          # t = -2 (3 + 1e-4) for every key but the first
    k[0, 0, 0] = 2.0           # E4M3 values: the row images keep them
    v[0, 0, 0] = 1.0
    scale = (3.0 + 1e-4) * np.log(2.0) / 2.0
    c = scale / np.log(2.0)
    qh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(q))
    kh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(k))
    t = c * (qh[:, 0] @ kh[:, 0].T)
    assert abs(t[0, 0] - 3.0 - 1e-4) < 1e-12
    assert 1e-4 < score_error(qh[:, 0], kh[:, 0], t, c)[0, 0]
    slack = fwd_slack(q, k, v, np.array([0, 1]), np.array([0, 32]), scale, False)
    den = np.exp2(t[0] - t[0].max()).sum()
    # key 0's weight: 256 2^(3 - 8 - t_max) under floor 3, 448 2^(2 - 8 - t_max) under floor 2
    assert slack[0, 0, 0] >= (1.0 - 448.0 / 512.0) * 2.0 ** (3.0 - t[0, 0]) / den - 1e-12
    # further from the integer than the bound: no allowance for key 0
    slack = fwd_slack(q, k, v, np.array([0, 1]), np.array([0, 32]), (3.0 + 1e-2) * np.log(2.0) / 2.0, False)
    assert slack[0, 0, 0] == 0.0


@pytest.mark.parametrize("rel", [1e-4, 1e-2])
def test_bwd_slack_covers_perturbed_p_and_ds(rel, monkeypatch):
    """The oracle's backward with every element of P and dS moved by up to
    rel of itself before its quantisation stays within bwd_slack (at
    eps_p = rel, eps_sum = 0) of the unperturbed gradients: the allowance
    goes through the right operand, axis and scale for dV, dK and dQ."""
    q, k, v, do, qo, ko = _draw([5, 37, 70, 0, 33], [5, 37, 70, 4, 60], 2, 64, 7, True)
    out, lse = mx.mx_attention_fwd(q, k, v, qo, ko, 0.3, True)
    ref = mx.mx_attention_bwd(q, k, v, out, do, lse, qo, ko, 0.3, True)
    slack = bwd_slack(q, k, v, out, do, lse, qo, ko, 0.3, True, eps_p=rel, eps_sum=0.0)
    rng = np.random.default_rng(8)
    orig = mx.mx_quantize_matrix
    monkeypatch.setattr(mx, "mx_quantize_matrix",
                        lambda x, axis: orig(x * (1 + rel * rng.choice([-1.0, 1.0, 0.0], x.shape) * rng.random(x.shape)),
                                             axis))
    moved = [0.0, 0.0, 0.0]
    for _ in range(4):
        got = mx.mx_attention_bwd(q, k, v, out, do, lse, qo, ko, 0.3, True)
        for i, (g, r, a) in enumerate(zip(got, ref, slack)):
            d = np.abs(g - r)
            assert np.all(d <= a + 1e-12), (i, np.max(d - a))
            moved[i] = max(moved[i], d.max())
    if rel >= 1e-3:
        assert min(moved) > 0   # the perturbations do flip decisions of P and of dS
