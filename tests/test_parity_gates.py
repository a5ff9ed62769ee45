"""The parity gates themselves, on the CPU: planted errors that the GPU tests
must reject.  A 20 % error confined to one 32-row tile of one sequence of a
12-sequence batch passes a whole-tensor relative L2 gate of 2e-2 but fails
the per-sequence gate; the bf16 forward bound is a flat 1e-2 below |out| = 2
and grows only by the output's own rounding above.  The bounds and floors
the gates add are checked here too: bf16 rounding reaches 2^-8 (the SiLU
weight and RoPE terms), the term-magnitude floor leaves a plain float32
backward passing and planted fp32 mistakes failing, and the term
magnitudes themselves equal scalar loops over every term."""

import math

import numpy as np
import pytest
import torch

from jagged_attention_ads_amd.workloads import offsets_from_lengths
from tests import gpu_util


def _grads(rng, lengths, H=4, d=64):
    off = offsets_from_lengths(lengths)
    T = int(off[-1])
    return off, [rng.standard_normal((T, H, d)) for _ in range(3)]


def _as_tensor(x):
    # float32 holds the planted values well inside the tolerances checked
    return torch.from_numpy(x.astype(np.float32))


def test_one_tile_error_fails_per_sequence_gate():
    rng = np.random.default_rng(5)
    lengths = list(rng.integers(200, 600, 12))
    off, refs = _grads(rng, lengths)
    bad = [r.copy() for r in refs]
    s0 = int(off[7]) + 64
    bad[0][s0:s0 + 32] *= 1.2            # dq: one 32-row tile of sequence 7 off by 20 %
    # the whole-tensor relative L2 error stays under 2e-2 ...
    assert gpu_util.rel_l2(bad[0], refs[0]) < gpu_util.GRAD_RTOL
    # ... while the per-sequence one does not
    worst, at = gpu_util.seq_rel_l2(bad[0], refs[0], off)
    assert at == 7 and worst > gpu_util.GRAD_RTOL
    grads = [_as_tensor(x).to(torch.bfloat16) for x in bad]
    # gated on tensors only, the planted error goes through (the bf16
    # storage of the values adds far less than the gate) ...
    gpu_util.check_backward(grads, refs)
    # ... gated per sequence, it is caught
    with pytest.raises(AssertionError, match="sequence 7"):
        gpu_util.check_backward(grads, refs, q_off=off, k_off=off)


def test_per_sequence_floor_for_cancelling_sequences():
    """A sequence whose reference gradient is (nearly) zero -- softmax with a
    single key gives dK = 0 exactly -- is measured against its share of the
    tensor's norm, not its own: tiny absolute errors there pass, a real
    error does not."""
    rng = np.random.default_rng(6)
    off, refs = _grads(rng, [50, 1, 80, 30])
    r = refs[1]
    r[int(off[1]):int(off[2])] = 0.0
    a = r + 1e-6 * rng.standard_normal(r.shape)
    worst, _ = gpu_util.seq_rel_l2(a, r, off)
    assert worst < 1e-3
    a[int(off[1]):int(off[2])] += 0.5
    worst, at = gpu_util.seq_rel_l2(a, r, off)
    assert at == 1 and worst > gpu_util.GRAD_RTOL


def test_per_sequence_gate_on_an_all_zero_gradient():
    """When the whole reference gradient is zero (every visible query sees a
    single key: dS = 0, so dq = dk = 0), there is no scale to be relative
    to, and the per-sequence error is the absolute norm, as the per-tensor
    one is: rounding-level values pass, real ones do not."""
    rng = np.random.default_rng(7)
    off = offsets_from_lengths([33, 60])
    r = np.zeros((93, 5, 128))
    a = 1e-7 * rng.standard_normal(r.shape)
    worst, _ = gpu_util.seq_rel_l2(a, r, off)
    assert worst == pytest.approx(max(np.linalg.norm(a[:33]), np.linalg.norm(a[33:])), rel=1e-12)
    assert worst < gpu_util.GRAD_RTOL_FP32
    assert gpu_util.rel_l2(a, r) == pytest.approx(np.linalg.norm(a))
    a[40:42] += 0.1
    worst, at = gpu_util.seq_rel_l2(a, r, off)
    assert at == 1 and worst > gpu_util.GRAD_RTOL


def test_silu_weight_rounding_bound():
    """The SiLU weight-rounding term: one key per query makes out = w v, so
    the bound is 2^-8 |w| |v| per element, exactly; masked (causal) and
    keyless rows get 0."""
    import dataclasses
    from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch
    wl = dataclasses.replace(WORKLOADS["gdpa_silu"], head_dim=32, heads=2, causal=True)
    b = make_batch(wl, 3, q_lengths=[4, 2], kv_lengths=[1, 0], with_dout=False)
    bound = gpu_util.silu_weight_rounding_of(b)
    q, k, v = b.f64("q"), b.f64("k"), b.f64("v")
    # sequence 0: 4 queries, one key; causal offset -3: only query 3 sees it
    assert not bound[:3].any() and not bound[4:].any()
    s = (q[3] * k[0]).sum(axis=-1) * b.scale               # [H]
    w = np.abs(s / (1.0 + np.exp(-s)))                      # L_kv = 1
    assert np.allclose(bound[3], 2.0 ** -8 * w[:, None] * np.abs(v[0]), rtol=1e-12, atol=0)


def test_bf16_rounding_reaches_two_to_the_minus_8():
    """The relative bound both rounding terms above use: bf16 keeps 8
    significant bits, so rounding to nearest moves a value by at most 2^-8
    of itself, and by more than 2^-9 just above a power of two (the weight
    4.0767 of a one-key SiLU row rounds to 4.0625)."""
    rng = np.random.default_rng(12)
    x = np.concatenate([rng.uniform(1.0, 2.0, 200000) * 2.0 ** rng.integers(-20, 20, 200000), [4.0767]])
    r = torch.from_numpy(x.astype(np.float32)).to(torch.bfloat16).double().numpy()
    rel = np.abs(r - x.astype(np.float32)) / np.abs(x.astype(np.float32))
    assert rel.max() <= 2.0 ** -8
    assert rel.max() > 0.99 * 2.0 ** -8 and rel[-1] > 2.0 ** -9


def test_forward_bound_flat_below_two():
    ref = np.array([0.0, 0.5, 1.99, 2.0, 3.9, 4.0, 7.9, -5.0])
    tol = gpu_util.forward_tolerance(ref, torch.bfloat16)
    assert np.all(tol[:3] == gpu_util.FWD_ATOL)
    # half a bf16 ulp: 2^-7 in [2, 4), 2^-6 in [4, 8) (taken at |ref| + 1e-2)
    assert tol[3] == pytest.approx(1e-2 + 2.0 ** -7)
    assert tol[4] == pytest.approx(1e-2 + 2.0 ** -7)   # 3.91 is still in [2, 4)
    assert tol[5] == pytest.approx(1e-2 + 2.0 ** -6)
    assert tol[7] == pytest.approx(1e-2 + 2.0 ** -6)
    assert np.all(gpu_util.forward_tolerance(ref, torch.float32) == gpu_util.FWD_ATOL_FP32)


def test_rope_lse_bound_covers_bf16_rounding_of_turned_inputs():
    """The lse bound for the fused rotary embedding holds for an emulation of
    exactly what it accounts for -- Q and K turned in fp64, rounded to bf16,
    then exact attention -- and is not loose by more than a few times."""
    import math
    import oracle
    rng = np.random.default_rng(8)
    lengths = [64, 30, 64, 5]
    off = offsets_from_lengths(lengths)
    T, H, d = int(off[-1]), 2, 64
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    s = 1.0 / math.sqrt(d)
    pos = oracle.sequence_positions(off) % 64
    as_bf16 = lambda x: torch.from_numpy(x).to(torch.bfloat16).double().numpy()  # noqa: E731
    qr, kr = as_bf16(oracle.rope(q, pos)), as_bf16(oracle.rope(k, pos))
    _, lse_em = oracle.attention_fwd(qr, kr, v, off, off, s, "softmax", True, block=64)
    _, lse_ref = oracle.attention_fwd(q, k, v, off, off, s, "softmax", True, block=64, rope_base=10000.0)
    bound = gpu_util.rope_lse_bound(q, k, off, 64, True, s) - gpu_util.LSE_ATOL
    err = np.abs(lse_em - lse_ref)
    assert np.all(err <= bound)
    assert err.max() > bound.max() / 50


def test_forward_bound_takes_the_ulp_where_the_value_can_reach():
    """With a per-element bound added (SiLU's weights), the unrounded value
    can cross into the next binade: the half-ulp is that binade's."""
    ref = np.array([1.995, 3.97, 1.5, 1.97])
    extra = np.array([0.02, 0.03, 0.0, 0.02])
    tol = gpu_util.forward_tolerance(ref, torch.bfloat16, extra)
    np.testing.assert_allclose(tol, [0.01 + 0.02 + 2.0 ** -7, 0.01 + 0.03 + 2.0 ** -6, 0.01, 0.01 + 0.02])


def _fp32_backward(q, k, v, do, qo, ko, scale, act, causal, p_to_bf16=False):
    """A plain float32 attention backward (the forward's O and lse too, in
    float32), to measure what ordinary fp32 rounding does against the fp64
    oracle.  p_to_bf16: round the weights to bf16 before the products (a
    mistake an fp32 path could make)."""
    from oracle.attention import visible_mask
    f = np.float32
    q, k, v, do = (x.astype(f) for x in (q, k, v, do))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    sc = f(scale)
    for b in range(len(qo) - 1):
        q0, q1, k0, k1 = int(qo[b]), int(qo[b + 1]), int(ko[b]), int(ko[b + 1])
        lq, lk = q1 - q0, k1 - k0
        if lq == 0 or lk == 0:
            continue
        vis = visible_mask(lq, lk, causal)
        for h in range(q.shape[1]):
            qs, ks, vs, ds = q[q0:q1, h], k[k0:k1, h], v[k0:k1, h], do[q0:q1, h]
            x = (qs @ ks.T) * sc
            dp = ds @ vs.T
            if act == "softmax":
                xm = np.where(vis, x, f(-np.inf))
                m = np.max(xm, axis=1, keepdims=True)
                with np.errstate(invalid="ignore"):   # rows that see no key: w = 0 below
                    lse = m + np.log(np.exp(xm - m).sum(axis=1, keepdims=True))
                w = np.where(vis, np.exp(xm - lse), f(0))
                o = w @ vs
                dsm = w * (dp - (ds * o).sum(axis=1, keepdims=True))
            else:
                sg = f(1) / (f(1) + np.exp(-x))
                w = np.where(vis, x * sg / f(lk), f(0))
                dsm = np.where(vis, sg * (f(1) + x * (f(1) - sg)) * dp / f(lk), f(0))
            if p_to_bf16:
                w = torch.from_numpy(np.ascontiguousarray(w)).to(torch.bfloat16).float().numpy()
            dv[k0:k1, h] = w.T @ ds
            dk[k0:k1, h] = (dsm.T @ qs) * sc
            dq[q0:q1, h] = (dsm @ ks) * sc
    return dq, dk, dv


@pytest.mark.parametrize("act,causal", [("softmax", False), ("softmax", True), ("silu", False), ("silu", True)])
def test_magnitude_floor(act, causal):
    """The per-sequence floor on the gradients' term magnitudes: a plain
    float32 backward passes the fp32 gate against the fp64 oracle in every
    sequence -- long ones, one key against many queries (softmax: dK = dQ =
    0 exactly, the float32 result is rounding residue) and cross lengths --
    and the floor is below the norm of every sequence whose gradient does
    not cancel, so it changes nothing there.  Mistakes an fp32 path could
    make still fail: the weights rounded to bf16, or the one-key sequence's
    cancellation broken (delta from a stale output)."""
    import oracle
    rng = np.random.default_rng(21)
    lq, lk = [300, 700, 1, 40, 513, 31], [300, 1, 1, 260, 513, 1]
    qo, ko = offsets_from_lengths(lq), offsets_from_lengths(lk)
    H, d = 2, 128
    q, do = (rng.standard_normal((int(qo[-1]), H, d)).astype(np.float32).astype(np.float64) for _ in range(2))
    k, v = (rng.standard_normal((int(ko[-1]), H, d)).astype(np.float32).astype(np.float64) for _ in range(2))
    scale = 1.0 / np.sqrt(d)
    ref = oracle.attention_bwd(q, k, v, do, qo, ko, scale, act, causal)
    mags = gpu_util.grad_term_magnitudes(q, k, v, do, qo, ko, scale, act, causal)
    got = _fp32_backward(q, k, v, do, qo, ko, scale, act, causal)
    worst = 0.0
    for g, r, m, off in zip(got, ref, mags, (qo, ko, ko)):
        w, _ = gpu_util.seq_rel_l2(g.astype(np.float64), r, off, m)
        worst = max(worst, w)
        for b in range(len(off) - 1):
            s0, s1 = int(off[b]), int(off[b + 1])
            rn = np.linalg.norm(r[s0:s1])
            if rn > 1e-8 * np.linalg.norm(m[s0:s1]):   # not cancelling
                assert gpu_util.MAG_FLOOR * np.linalg.norm(m[s0:s1]) < rn
    assert worst < 0.1 * gpu_util.GRAD_RTOL_FP32
    bad = _fp32_backward(q, k, v, do, qo, ko, scale, act, causal, p_to_bf16=True)
    assert max(gpu_util.seq_rel_l2(g.astype(np.float64), r, off, m)[0]
               for g, r, m, off in zip(bad, ref, mags, (qo, ko, ko))) > 2 * gpu_util.GRAD_RTOL_FP32
    if act == "softmax" and not causal:
        # sequence 1: 700 queries, one key; delta taken from out 1e-3 off
        bad = [x.copy() for x in got]
        s0, s1 = int(qo[1]), int(qo[2])
        delta_err = 1e-3 * (do[s0:s1] * v[int(ko[1])]).sum(axis=-1)          # [700, H]
        bad[1][int(ko[1])] -= scale * (delta_err[..., None] * q[s0:s1]).sum(axis=0)
        w, at = gpu_util.seq_rel_l2(bad[1].astype(np.float64), ref[1], ko, mags[1])
        assert at == 1 and w > 2 * gpu_util.GRAD_RTOL_FP32


@pytest.mark.parametrize("act,causal", [("softmax", False), ("softmax", True), ("silu", True)])
def test_grad_term_magnitudes_brute_force(act, causal):
    """grad_term_magnitudes against scalar loops over every term, written
    from the gradients' definitions (softmax: dS = P dP - P delta, its two
    parts apart; SiLU: dS = silu'(x) dP / L_kv), on tiny cross-length
    sequences (causal: key j visible to query i when j <= i + L_kv - L_q)."""
    rng = np.random.default_rng(31)
    lq, lk = [3, 1, 4], [5, 2, 4]
    qo, ko = offsets_from_lengths(lq), offsets_from_lengths(lk)
    H, d, scale = 2, 4, 0.7
    q, do = (rng.standard_normal((int(qo[-1]), H, d)) for _ in range(2))
    k, v = (rng.standard_normal((int(ko[-1]), H, d)) for _ in range(2))
    mq, mk, mv = gpu_util.grad_term_magnitudes(q, k, v, do, qo, ko, scale, act, causal)
    eq, ek, ev = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(lq)):
        for h in range(H):
            for i in range(lq[b]):
                qi = int(qo[b]) + i
                keys = [j for j in range(lk[b]) if not causal or j <= i + lk[b] - lq[b]]
                x = {j: scale * sum(q[qi, h, c] * k[int(ko[b]) + j, h, c] for c in range(d)) for j in keys}
                dp = {j: sum(do[qi, h, c] * v[int(ko[b]) + j, h, c] for c in range(d)) for j in keys}
                if act == "softmax":
                    z = sum(math.exp(x[j]) for j in keys)
                    p = {j: math.exp(x[j]) / z for j in keys}
                    o = [sum(p[j] * v[int(ko[b]) + j, h, c] for j in keys) for c in range(d)]
                    delta = sum(do[qi, h, c] * o[c] for c in range(d))
                    w = p
                    t = {j: p[j] * abs(dp[j]) + p[j] * abs(delta) for j in keys}
                else:
                    sg = {j: 1.0 / (1.0 + math.exp(-x[j])) for j in keys}
                    w = {j: abs(x[j] * sg[j]) / lk[b] for j in keys}
                    t = {j: abs(sg[j] * (1 + x[j] * (1 - sg[j])) * dp[j]) / lk[b] for j in keys}
                for j in keys:
                    kj = int(ko[b]) + j
                    for c in range(d):
                        ev[kj, h, c] += abs(w[j]) * abs(do[qi, h, c])
                        ek[kj, h, c] += scale * t[j] * abs(q[qi, h, c])
                        eq[qi, h, c] += scale * t[j] * abs(k[kj, h, c])
    for got, exp in ((mq, eq), (mk, ek), (mv, ev)):
        np.testing.assert_allclose(got, exp, rtol=1e-12, atol=1e-15)


@pytest.mark.parametrize("causal,block", [(True, 64), (False, 35)])
def test_rope_rounding_effect_within_its_first_order_bound(causal, block):
    """rope_rounding_effect (the output change from rounding the turned Q
    and K to bf16) against the bound that score errors |ds_ij| <= e_ij
    imply for a softmax output to first order,
      |d out_ic| <= sum_j p_ij (e_ij + sum_k p_ik e_ik) |v_jc - out_ic|,
    with e_ij = scale 2^-7 sum over rotation pairs of the pair lengths of q_i
    and k_j (each rounding moves a turned value by at most 2^-8 of itself;
    a turn keeps pair lengths).  The effect is nonzero and within the bound,
    and the bound is not loose by orders of magnitude."""
    import oracle
    from oracle.attention import visible_mask
    rng = np.random.default_rng(41)
    lengths = [64, 30, 100, 5]
    off = offsets_from_lengths(lengths)
    T, H, d = int(off[-1]), 2, 64
    q, k, v = (rng.standard_normal((T, H, d)) for _ in range(3))
    s = 1.0 / np.sqrt(d)
    eff = gpu_util.rope_rounding_effect(q, k, v, off, block, s, "softmax", causal, 10000.0)
    out, _ = oracle.attention_fwd(q, k, v, off, off, s, "softmax", causal, block=block, rope_base=10000.0)
    h2 = d // 2
    qn = np.sqrt(q[..., :h2] ** 2 + q[..., h2:] ** 2)
    kn = np.sqrt(k[..., :h2] ** 2 + k[..., h2:] ** 2)
    bound = np.zeros_like(eff)
    for b in range(len(lengths)):
        for c0 in range(int(off[b]), int(off[b + 1]), block):
            c1 = min(c0 + block, int(off[b + 1]))
            vis = visible_mask(c1 - c0, c1 - c0, causal)
            for h in range(H):
                from oracle.rope import rope as turn
                pos = np.arange(c1 - c0)
                qt, kt = turn(q[c0:c1, h:h + 1], pos)[:, 0], turn(k[c0:c1, h:h + 1], pos)[:, 0]
                x = np.where(vis, s * (qt @ kt.T), -np.inf)
                p = np.exp(x - x.max(axis=1, keepdims=True))
                p /= p.sum(axis=1, keepdims=True)
                e = s * 2.0 ** -7 * (qn[c0:c1, h] @ kn[c0:c1, h].T)
                w = p * (e + (p * e).sum(axis=1, keepdims=True))
                vv = v[c0:c1, h]
                o = out[c0:c1, h]
                bound[c0:c1, h] = np.einsum("ij,ijc->ic", w, np.abs(vv[None, :, :] - o[:, None, :]))
    assert eff.max() > 0
    assert np.all(eff <= bound * (1 + 1e-3) + 1e-12)
    assert eff.max() > bound.max() / 100
