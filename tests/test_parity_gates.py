"""The parity gates themselves, on the CPU: planted errors that the GPU tests
must reject.  A 20 % error confined to one 32-row tile of one sequence of a
12-sequence batch passes a whole-tensor relative L2 gate of 2e-2 but fails
the per-sequence gate; the bf16 forward bound is a flat 1e-2 below |out| = 2
and grows only by the output's own rounding above."""

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
    the bound is 2^-9 |w| |v| per element, exactly; masked (causal) and
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
    assert np.allclose(bound[3], 2.0 ** -9 * w[:, None] * np.abs(v[0]), rtol=1e-12, atol=0)


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
