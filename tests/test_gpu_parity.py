"""Parity of the HIP path (through the C ABI) with the fp64 CPU oracle.

Gates (bf16): forward abs error <= 1e-2 per element where |out| < 2, and
1e-2 plus half a bf16 ulp of |out| above (the stored output's own rounding);
lse abs error <= 1e-3 (lse = -inf exactly where the oracle has no visible
key); relative L2 error of dq, dk, dv <= 2e-2, per tensor and per sequence.
fp32 inputs: 1e-4 for the forward and for the gradients.
"""

import dataclasses

import numpy as np
import pytest
import torch

from jagged_attention_ads_amd.workloads import ORDER, WORKLOADS, make_batch
from tests.gpu_util import (Dev, check_backward, check_forward, oracle_bwd, oracle_fwd, rows_of, seq_offsets)

pytestmark = pytest.mark.gpu

# reduced batches: several tiles per sequence and ragged tails, oracle in seconds
REDUCED = [("tiny_fp32", None), ("selfattn_causal", 12), ("cross_asym", 24), ("gdpa_silu", 6),
           ("pareto_train", 96)]


def _seed(name):
    return ORDER.index(name) + 1


@pytest.mark.parametrize("name,batch", REDUCED)
def test_forward_reduced(name, batch):
    b = make_batch(name, _seed(name), batch=batch)
    d = Dev(b)
    out, lse = d.forward()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_fwd(b)
    check_forward(out, lse, ref_out, ref_lse, b.workload.activation)


@pytest.mark.parametrize("name,batch", [x for x in REDUCED if WORKLOADS[x[0]].backward])
def test_backward_reduced(name, batch):
    b = make_batch(name, _seed(name), batch=batch)
    d = Dev(b)
    out, lse = d.forward()
    grads = d.backward(out, lse)
    torch.cuda.synchronize()
    check_backward(grads, oracle_bwd(b), q_off=b.q_offsets, k_off=b.kv_offsets)


# ------------------------------------------------------------------ edge cases

EDGE = {
    # name: (base workload, q lengths, kv lengths, overrides)
    "empty_seqs": ("selfattn_causal", [0, 5, 130, 0, 1, 64], [3, 0, 130, 0, 1, 64], dict(causal=False)),
    "empty_seqs_causal": ("selfattn_causal", [0, 5, 130, 0, 1, 64], [3, 0, 130, 0, 1, 64], {}),
    "cross_causal_q_longer": ("selfattn_causal", [200, 70, 9], [64, 3, 9], dict(head_dim=64)),
    "cross_causal_k_longer": ("selfattn_causal", [5, 65, 128], [300, 129, 1000], dict(head_dim=64)),
    "tile_boundaries": ("selfattn_causal", [1, 63, 64, 65, 127, 128, 129, 255, 256, 257],
                        [1, 63, 64, 65, 127, 128, 129, 255, 256, 257], {}),
    "long_noncausal": ("selfattn_causal", [700, 1030], [1030, 700], dict(causal=False)),
    "d32_silu_causal": ("gdpa_silu", [40, 130, 7], [40, 130, 7], dict(head_dim=32)),
    "d64_silu_cross": ("gdpa_silu", [33, 1, 100], [200, 17, 64], dict(head_dim=64, causal=False)),
    "d64_fp32_softmax": ("tiny_fp32", [70, 3, 129], [70, 3, 129], dict(head_dim=64, causal=True)),
    "d128_fp32_silu": ("tiny_fp32", [20, 66], [33, 66], dict(head_dim=128, activation="silu")),
    "d32_bf16_cross": ("cross_asym", [1, 64, 17], [4096, 5, 300], dict(head_dim=32, heads=3)),
    "many_heads": ("selfattn_causal", [50, 130], [50, 130], dict(heads=16, head_dim=64)),
    # the dQ pass over stored dS takes 256-row items when no sequence is much
    # longer than the mean (max <= 4 x mean, max > 128), 128-row items otherwise
    "dq_items_256": ("selfattn_causal", [300, 260, 290, 129], [300, 260, 290, 129], {}),
    "dq_items_128": ("selfattn_causal", [900] + [5] * 20, [900] + [5] * 20, {}),
    # the largest key length the scheduler accepts (1023 cost classes of 64 keys)
    "max_kv_len": ("cross_asym", [64, 3], [65472, 1000], dict(heads=2)),
    # the largest head count (the head index is packed into 8 bits of an item)
    "max_heads": ("selfattn_causal", [3, 40], [3, 40], dict(heads=256, head_dim=32)),
}


def _edge_batch(name):
    base, lq, lk, over = EDGE[name]
    wl = dataclasses.replace(WORKLOADS[base], backward=True, **over)
    return make_batch(wl, 100 + sorted(EDGE).index(name), q_lengths=lq, kv_lengths=lk, with_dout=True)


@pytest.fixture(params=["stored_ds", "recompute", "short_in_dkdv"])
def dq_path(request, options):
    """The backward's dQ paths: from the dS blocks the dK/dV pass stores (the
    default), or recomputing dS (option bwd_ds_store off; also what runs when
    the dS store would not fit the workspace limit).  short_in_dkdv (option
    bwd_short_dq on) has the dK/dV pass write the dQ of the short sequences
    (<= 64 queries, 1 .. 64 keys) in any batch, not only in one where every
    sequence is short, and the dQ pass skip them."""
    if request.param == "recompute":
        options("bwd_ds_store", 0)
    elif request.param == "short_in_dkdv":
        options("bwd_short_dq", 1)
    return request.param


@pytest.mark.parametrize("name,batch", [x for x in REDUCED if WORKLOADS[x[0]].backward])
def test_backward_reduced_recompute(name, batch, options):
    options("bwd_ds_store", 0)
    b = make_batch(name, _seed(name), batch=batch)
    d = Dev(b)
    out, lse = d.forward()
    grads = d.backward(out, lse)
    torch.cuda.synchronize()
    check_backward(grads, oracle_bwd(b), q_off=b.q_offsets, k_off=b.kv_offsets)


def test_backward_small_workspace_recomputes():
    """A workspace without the dS store (for_backward = 2) is accepted and
    gives the recomputing dQ pass: results within the gates, and dK, dV
    bitwise equal to the full workspace's (the dK/dV pass is the same)."""
    from jagged_attention_ads_amd import jfa
    b = make_batch("selfattn_causal", _seed("selfattn_causal"), batch=12)
    d = Dev(b)
    out, lse = d.forward()
    T_q, H, D = d.q.shape
    B = len(b.q_lengths)
    full = jfa.workspace(B, H, D, T_q, d.k.shape[0], d.mk, d.q.dtype, 1, d.q.device)
    small = jfa.workspace(B, H, D, T_q, d.k.shape[0], d.mk, d.q.dtype, 2, d.q.device)
    assert small.numel() < full.numel()
    g_full = jfa.backward(d.q, d.k, d.v, out, d.do, lse, d.qo, d.ko, d.mq, d.mk, d.scale, d.act, d.causal, ws=full)
    g_small = jfa.backward(d.q, d.k, d.v, out, d.do, lse, d.qo, d.ko, d.mq, d.mk, d.scale, d.act, d.causal, ws=small)
    torch.cuda.synchronize()
    ref = oracle_bwd(b)
    check_backward(g_full, ref, q_off=b.q_offsets, k_off=b.kv_offsets)
    check_backward(g_small, ref, q_off=b.q_offsets, k_off=b.kv_offsets)
    for x, y in zip(g_full[1:], g_small[1:]):
        assert torch.equal(x.view(torch.int16), y.view(torch.int16))


@pytest.mark.parametrize("name", sorted(EDGE))
def test_edge_cases(name, dq_path):
    b = _edge_batch(name)
    d = Dev(b)
    out, lse = d.forward()
    grads = d.backward(out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_fwd(b)
    check_forward(out, lse, ref_out, ref_lse, b.workload.activation)
    check_backward(grads, oracle_bwd(b), q_off=b.q_offsets, k_off=b.kv_offsets)


# ------------------------------------------------------------------ short sequences

# Short sequences (at most 64 queries and 1 .. 64 keys) are one dK/dV item each;
# that item can also write their dQ, and the dQ pass then skips them.  It does
# by default when every sequence is short (or has no keys): the dQ pass only
# zeroes the rows of sequences without keys.  In mixed batches it does with
# option bwd_short_dq on: short sequences next to ones the dQ pass takes, ones
# with no keys or no queries, and causal cases where the first query block
# sees no key (64 queries, 10 keys).
SHORT_Q = [1, 31, 32, 33, 63, 64, 64, 40, 0, 7, 300, 64, 17]
SHORT_K = [1, 31, 32, 33, 63, 64, 10, 20, 5, 0, 300, 65, 64]
ALL_SHORT_Q = [1, 64, 40, 7, 0, 33, 64, 12]
ALL_SHORT_K = [1, 10, 64, 0, 5, 33, 64, 0]
SHORT = {
    "softmax_causal": ("selfattn_causal", {}, SHORT_Q, SHORT_K),
    "softmax_noncausal": ("selfattn_causal", dict(causal=False), SHORT_Q, SHORT_K),
    "silu_causal_d64": ("gdpa_silu", dict(head_dim=64), SHORT_Q, SHORT_K),
    "softmax_noncausal_d64": ("cross_asym", dict(heads=3), SHORT_Q, SHORT_K),
    "all_short_causal": ("selfattn_causal", {}, ALL_SHORT_Q, ALL_SHORT_K),
    "all_short_silu": ("gdpa_silu", dict(causal=False), ALL_SHORT_Q, ALL_SHORT_K),
    # no room for the fused dQ in these dK/dV kernels: two passes, while the
    # forward still takes its two-wave variant
    "all_short_fp32_d128": ("tiny_fp32", dict(head_dim=128, causal=True), ALL_SHORT_Q, ALL_SHORT_K),
    "all_short_bf16_d32": ("selfattn_causal", dict(head_dim=32, heads=3), ALL_SHORT_Q, ALL_SHORT_K),
}


@pytest.mark.parametrize("name", sorted(SHORT))
def test_short_sequences_dq_in_dkdv(name, options):
    """Within the gates of the oracle, and bitwise equal to the results with
    the short sequences left to the dQ pass over stored dS: both take the
    same dS blocks and sum the same products in the same order."""
    base, over, lq, lk = SHORT[name]
    wl = dataclasses.replace(WORKLOADS[base], backward=True, **over)
    b = make_batch(wl, 200 + sorted(SHORT).index(name), q_lengths=lq, kv_lengths=lk, with_dout=True)
    d = Dev(b)
    if max(lq) > 64 or max(lk) > 64:
        options("bwd_short_dq", 1)
    out, lse = d.forward()
    fused = d.backward(out, lse)
    options("bwd_short_dq", 0)
    apart = d.backward(out, lse)
    torch.cuda.synchronize()
    check_backward(fused, oracle_bwd(b), q_off=b.q_offsets, k_off=b.kv_offsets)
    for x, y in zip(fused, apart):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


@pytest.mark.parametrize("name", [n for n in sorted(SHORT) if n.startswith("all_short")])
def test_short_batch_forward_variant(name, options):
    """A batch whose sequences all have at most 64 queries and keys runs the
    two-wave forward variant: within the gates of the oracle, and bitwise
    equal to the four-wave kernel (option fwd_short off), whose per-row
    arithmetic it shares."""
    base, over, lq, lk = SHORT[name]
    wl = dataclasses.replace(WORKLOADS[base], **over)
    b = make_batch(wl, 300 + sorted(SHORT).index(name), q_lengths=lq, kv_lengths=lk, with_dout=False)
    d = Dev(b)
    out, lse = d.forward()
    options("fwd_short", 0)
    out4, lse4 = d.forward()
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_fwd(b)
    check_forward(out, lse, ref_out, ref_lse, b.workload.activation)
    assert torch.equal(out.view(torch.uint8), out4.view(torch.uint8))
    if lse is not None:
        assert torch.equal(lse.view(torch.int32), lse4.view(torch.int32))


# ------------------------------------------------------------------ full sizes, sampled

def _sample(b, rng, n=3):
    lens = b.q_lengths * np.maximum(b.kv_lengths, 1)
    pick = {int(np.argmax(lens)), int(np.argmin(b.q_lengths + (b.q_lengths == 0) * 10**9))}
    pick |= set(int(x) for x in rng.choice(len(lens), size=n, replace=False))
    return sorted(pick)


@pytest.mark.parametrize("name", ORDER)
def test_full_size_sampled(name):
    """Full-size batches, as the benchmark runs them: every output row comes
    from the batched launch; the oracle recomputes sampled sequences alone
    (sequences are independent)."""
    b = make_batch(name, _seed(name))
    d = Dev(b)
    out, lse = d.forward()
    grads = d.backward(out, lse) if b.workload.backward else None
    torch.cuda.synchronize()
    seqs = _sample(b, np.random.default_rng(_seed(name)))
    qr, kr = rows_of(b, seqs, "q"), rows_of(b, seqs, "k")
    ref_out, ref_lse = oracle_fwd(b, seqs)
    check_forward(out, lse, ref_out, ref_lse, b.workload.activation, q_rows=qr)
    if grads is not None:
        qso, kso = seq_offsets(b, seqs)
        check_backward(grads, oracle_bwd(b, seqs), q_rows=qr, k_rows=kr, q_off=qso, k_off=kso)
    # every row of the full outputs is finite (no row was skipped or left unwritten)
    assert torch.isfinite(out).all()
    if grads is not None:
        for g in grads:
            assert torch.isfinite(g).all()

