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
