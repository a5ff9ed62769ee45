"""Seeded random configurations of the bf16 / fp32 path against the fp64
oracle, forward and backward, with the gates of test_gpu_parity.

Each case draws, from its own seed: the element type, head_dim (32, 64,
128), the head count, softmax or SiLU, causal or not, self- or
cross-attention, 1 to 9 sequences whose lengths mix empty sequences, single
tokens, lengths one off a tile boundary (31 .. 257) and uniform ones up to
300, and one of the backward's three dQ paths.  The edge-case tests pin the
boundaries one at a time; these cases combine them.
"""

import dataclasses

import numpy as np
import pytest
import torch

from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch
from tests.gpu_util import Dev, check_backward, check_forward, oracle_bwd, oracle_fwd, silu_weight_rounding

pytestmark = pytest.mark.gpu

BOUNDARY = [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
N_CASES = 64


def _length(rng):
    kind = rng.integers(0, 6)
    if kind == 0:
        return 0
    if kind == 1:
        return 1
    if kind in (2, 3):
        return int(rng.choice(BOUNDARY))
    return int(rng.integers(2, 301))


def _config(case):
    rng = np.random.default_rng(7000 + case)
    fp32 = rng.random() < 0.25
    d = int(rng.choice([32, 64, 128]))
    heads = int(rng.choice([1, 2, 3, 5, 8]))
    act = "silu" if rng.random() < 0.35 else "softmax"
    causal = bool(rng.random() < 0.5)
    cross = bool(rng.random() < 0.4)
    n = int(rng.integers(1, 10))
    lq = [_length(rng) for _ in range(n)]
    lk = [_length(rng) for _ in range(n)] if cross else list(lq)
    path = ["stored_ds", "recompute", "short_in_dkdv"][int(rng.integers(0, 3))]
    base = "tiny_fp32" if fp32 else "selfattn_causal"
    wl = dataclasses.replace(WORKLOADS[base], head_dim=d, heads=heads, activation=act, causal=causal, backward=True)
    return wl, lq, lk, path


@pytest.mark.parametrize("case", range(N_CASES))
def test_random_configuration(case, options):
    wl, lq, lk, path = _config(case)
    print("case %d: %s d %d heads %d %s causal %s q %s kv %s dq path %s" % (
        case, wl.dtype, wl.head_dim, wl.heads, wl.activation, wl.causal, lq, lk, path), flush=True)
    if path == "recompute":
        options("bwd_ds_store", 0)
    elif path == "short_in_dkdv":
        options("bwd_short_dq", 1)
    b = make_batch(wl, 7100 + case, q_lengths=lq, kv_lengths=lk, with_dout=True)
    d = Dev(b)
    out, lse = d.forward()
    grads = d.backward(out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_fwd(b)
    # SiLU's weights are not normalised: their bf16 rounding moves the output
    # by up to 2^-9 of sum |w| |v| (tests.gpu_util.silu_weight_rounding)
    extra = silu_weight_rounding(b) if wl.activation == "silu" and wl.dtype == "bf16" else None
    check_forward(out, lse, ref_out, ref_lse, wl.activation, extra_tol=extra)
    check_backward(grads, oracle_bwd(b), q_off=b.q_offsets, k_off=b.kv_offsets)
    # rows of sequences that see no key get zero dq; keys no query sees get
    # zero dk and dv
    for s in np.nonzero(b.kv_lengths == 0)[0]:
        assert not (grads[0][int(b.q_offsets[s]):int(b.q_offsets[s + 1])] != 0).any()
    for s in np.nonzero(b.q_lengths == 0)[0]:
        for g in grads[1:]:
            assert not (g[int(b.kv_offsets[s]):int(b.kv_offsets[s + 1])] != 0).any()
