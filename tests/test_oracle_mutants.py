"""The pins catch plausible mistakes: each test plants one mistake in a copy of
the oracle's arithmetic (on the CPU) and checks that an independent pin
(brute force, torch SDPA, a closed form or finite differences) rejects it.
"""

import math

import numpy as np
import pytest

import oracle
import oracle.attention as A
from tests.test_oracle_pins import brute_force_fwd, _draw, _sdpa_per_sequence


def _mask_off_by_one(lq, lk, causal):
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return (j < i + (lk - lq)) if causal else np.ones((lq, lk), bool)


def _mask_top_left(lq, lk, causal):
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    return (j <= i) if causal else np.ones((lq, lk), bool)


def _sigmoid_wrong_sign(x):
    return 1.0 / (1.0 + np.exp(x))


def _fwd_mismatch(monkeypatch, activation, causal, qlen, klen):
    q, k, v, _, qo, ko = _draw(qlen, klen, 2, 3, seed=21)
    out, _ = oracle.attention_fwd(q, k, v, qo, ko, 0.5, activation, causal)
    monkeypatch.undo()
    ref, _ = brute_force_fwd(q, k, v, qo, ko, 0.5, activation, causal)
    return np.abs(out - ref).max()


@pytest.mark.parametrize("mutant", [_mask_off_by_one, _mask_top_left])
def test_mask_mistakes_are_caught(monkeypatch, mutant):
    monkeypatch.setattr(A, "visible_mask", mutant)
    assert _fwd_mismatch(monkeypatch, "softmax", True, [3, 5], [6, 5]) > 1e-3


def test_sigmoid_sign_mistake_is_caught(monkeypatch):
    monkeypatch.setattr(A, "_sigmoid", _sigmoid_wrong_sign)
    assert _fwd_mismatch(monkeypatch, "silu", False, [3, 4], [4, 2]) > 1e-3


def test_dropped_silu_normaliser_is_caught(monkeypatch):
    orig = A._probs

    def no_norm(S, vis, activation, lk):
        P, lse = orig(S, vis, activation, lk)
        return (P * lk, lse) if activation == "silu" else (P, lse)
    monkeypatch.setattr(A, "_probs", no_norm)
    assert _fwd_mismatch(monkeypatch, "silu", True, [3, 4], [3, 4]) > 1e-3


def test_transposed_backward_operand_is_caught(monkeypatch):
    """dK computed as scale * dS^T K instead of scale * dS^T Q (shape-valid
    when Lq == Lk) must disagree with torch autograd."""
    q, k, v, do, qo, ko = _draw([4, 6], [4, 6], 2, 3, seed=22)
    orig_bwd = A.attention_bwd

    def bad_bwd(q, k, v, dout, q_offsets, kv_offsets, scale, activation="softmax", causal=False):
        dq, dk, dv = orig_bwd(q, k, v, dout, q_offsets, kv_offsets, scale, activation, causal)
        # recompute dk with K in place of Q for every block
        for b in range(len(q_offsets) - 1):
            qs, qe, ks, ke = q_offsets[b], q_offsets[b + 1], kv_offsets[b], kv_offsets[b + 1]
            for h in range(q.shape[1]):
                S = scale * q[qs:qe, h] @ k[ks:ke, h].T
                P, _ = A._probs(S, A.visible_mask(qe - qs, ke - ks, causal), activation, ke - ks)
                dP = dout[qs:qe, h] @ v[ks:ke, h].T
                dS = P * (dP - (P * dP).sum(1, keepdims=True))
                dk[ks:ke, h] = scale * dS.T @ k[ks:ke, h]
        return dq, dk, dv
    _, dk_bad, _ = bad_bwd(q, k, v, do, qo, ko, 0.5, "softmax", False)
    _, _, r_dk, _ = _sdpa_per_sequence(q, k, v, do, qo, ko, 0.5, False)
    assert np.abs(dk_bad - r_dk).max() > 1e-3
    _, dk_good, _ = A.attention_bwd(q, k, v, do, qo, ko, 0.5, "softmax", False)
    assert np.abs(dk_good - r_dk).max() < 1e-12


def test_wrong_silu_derivative_is_caught(monkeypatch):
    """silu'(x) = sig(x)(1 + x(1 - sig(x))); dropping the x-term must fail
    the finite-difference check."""
    q, k, v, do, qo, ko = _draw([3], [4], 1, 2, seed=23)
    s = 0.9

    def loss(qq):
        return float((oracle.attention_fwd(qq, k, v, qo, ko, s, "silu", False)[0] * do).sum())
    h = 1e-6
    num = np.zeros_like(q)
    for idx in np.ndindex(q.shape):
        p, m = q.copy(), q.copy()
        p[idx] += h
        m[idx] -= h
        num[idx] = (loss(p) - loss(m)) / (2 * h)
    # the planted mistake, written out: derivative sig(x) only
    S = s * q[:, 0] @ k[:, 0].T
    sig = 1 / (1 + np.exp(-S))
    dA = do[:, 0] @ v[:, 0].T
    dq_bad = s * (dA * sig / 4) @ k[:, 0]
    assert np.linalg.norm(dq_bad - num[:, 0]) / np.linalg.norm(num) > 1e-3
    dq_good = oracle.attention_bwd(q, k, v, do, qo, ko, s, "silu", False)[0]
    assert np.linalg.norm(dq_good - num) / np.linalg.norm(num) < 1e-6


def test_lse_base_mistake_is_caught():
    """lse stored in log2 instead of ln would fail the golden closed form."""
    q = np.array([[[1.0]]])
    k = np.array([[[0.0]], [[math.log(3)]]])
    v = np.array([[[4.0]], [[8.0]]])
    _, lse = oracle.attention_fwd(q, k, v, [0, 1], [0, 2], 1.0, "softmax", False)
    assert abs(lse[0, 0] - math.log(4)) < 1e-14
    assert abs(lse[0, 0] / math.log(2) - math.log(4)) > 0.1


def _segments_shifted(qo, ko, block):
    """Blocks counted from the second token of each sequence instead of its first."""
    segs = []
    for b in range(len(qo) - 1):
        qs, qe = qo[b], qo[b + 1]
        cuts = [qs] + list(range(qs + 1, qe, block)) + [qe] if qe - qs > 1 else [qs, qe]
        cuts = sorted(set(cuts))
        segs += [(x, y, x - qs + ko[b], y - qs + ko[b]) for x, y in zip(cuts[:-1], cuts[1:])]
    return segs


def _segments_sequence_normaliser(qo, ko, block):
    """Blocks right, but a mistake of the GDPA normaliser: its units are the
    whole sequences (the blocks' masks are lost)."""
    return [(qo[b], qo[b + 1], ko[b], ko[b + 1]) for b in range(len(qo) - 1)]


@pytest.mark.parametrize("mutant", [_segments_shifted, _segments_sequence_normaliser])
@pytest.mark.parametrize("activation", ["softmax", "silu"])
def test_block_mistakes_are_caught(monkeypatch, mutant, activation):
    from tests.test_oracle_pins import brute_force_block_fwd
    lens = [7, 3, 9]
    q, k, v, _, qo, _ = _draw(lens, lens, 2, 3, seed=44)
    monkeypatch.setattr(A, "_segments", mutant)
    out, _ = oracle.attention_fwd(q, k, v, qo, qo, 0.6, activation, True, block=3)
    monkeypatch.undo()
    ref, _ = brute_force_block_fwd(q, k, v, qo, 0.6, activation, True, 3)
    assert np.abs(out - ref).max() > 1e-3


# ------------------------------------------------------------------ MXFP8


def _mx_loop_mismatch(monkeypatch, causal=True):
    from tests.test_oracle_mx import _loop_mx_attention
    import oracle.mx as mx
    rng = np.random.default_rng(31)
    lq, lk = [3, 36], [40, 36]
    qo = np.concatenate([[0], np.cumsum(lq)])
    ko = np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((qo[-1], 1, 32)) * 2
    k = rng.standard_normal((ko[-1], 1, 32))
    v = rng.standard_normal((ko[-1], 1, 32)) * np.exp2(rng.integers(-5, 5, (ko[-1], 1, 32)))
    out, _ = mx.mx_attention_fwd(q, k, v, qo, ko, 0.4, causal)
    monkeypatch.undo()
    ref, _ = _loop_mx_attention(q, k, v, qo, ko, 0.4, causal)
    return np.abs(out - ref).max()


def test_mx_global_block_alignment_is_caught(monkeypatch):
    import oracle.mx as mx
    orig = mx.mx_quantize_keys

    def global_blocks(x, offsets):
        return orig(x, [0, np.asarray(x).shape[0]])   # blocks counted from row 0 of the packed tensor
    monkeypatch.setattr(mx, "mx_quantize_keys", global_blocks)
    assert _mx_loop_mismatch(monkeypatch) > 1e-6


def test_mx_p_scale_from_rounded_max_is_caught(monkeypatch):
    import oracle.mx as mx
    orig_floor = np.floor

    def quantize_p_round(t, vis):
        monkeypatch.setattr(mx.np, "floor", np.round)
        try:
            return mx_quantize_p(t, vis)
        finally:
            monkeypatch.setattr(mx.np, "floor", orig_floor)
    mx_quantize_p = mx.quantize_p
    monkeypatch.setattr(mx, "quantize_p", quantize_p_round)
    assert _mx_loop_mismatch(monkeypatch) > 1e-6


def test_mx_quantised_denominator_is_caught():
    import json
    import os
    import oracle.mx as mx
    cases = json.load(open(os.path.join(os.path.dirname(__file__), "golden", "mx_cases.json")))
    e = cases["p_examples"][0]
    t = np.array(e["t"])
    codes, fb = mx.quantize_p(t[None, :], np.ones((1, len(t)), bool))
    w = mx.e4m3_decode(codes[0]) * 2.0 ** (fb[0, 0] - 8)
    wrong = w / w.sum()          # normalised by the quantised weights instead of the exact ones
    assert np.abs(wrong - np.array(e["out"])).max() > 1e-3


def test_mx_backward_wrong_quantisation_axis_is_caught(monkeypatch):
    """dS quantised along keys for every product (instead of along queries
    for dK and dV's P): the loop implementation rejects it."""
    from tests.test_oracle_mx import _draw_bwd, _loop_mx_bwd
    import oracle.mx as mx
    q, k, v, out, do, lse, qo, ko = _draw_bwd([2, 35], [36, 33], 1, 32, 5, False)
    orig = mx.mx_quantize_matrix
    monkeypatch.setattr(mx, "mx_quantize_matrix", lambda x, axis: orig(x, 1))
    got = mx.mx_attention_bwd(q, k, v, out, do, lse, qo, ko, 0.3, False)
    monkeypatch.undo()
    ref = _loop_mx_bwd(q, k, v, out, do, lse, qo, ko, 0.3, False)
    assert max(np.abs(g - r).max() for g, r in zip(got, ref)) > 1e-6
