"""Seeded random configurations of the bf16 / fp32 path against the fp64
oracle, forward and backward, with the gates of test_gpu_parity.

Each case draws, from its own seed: the element type, head_dim (32, 64,
128), the head count, softmax or SiLU, causal or not, self- or
cross-attention, 1 to 9 sequences whose lengths mix empty sequences, single
tokens, lengths one off a tile boundary (31 .. 257) and uniform ones up to
300, and one of the backward's three dQ paths.  The edge-case tests pin the
boundaries one at a time; these cases combine them.  Twelve more take 1 to 3
sequences of up to 3000 tokens.
"""

import dataclasses

import numpy as np
import pytest
import torch

from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch
from tests.gpu_util import (Dev, check_backward, check_forward, grad_term_magnitudes, grad_term_magnitudes_of,
                            oracle_bwd, oracle_fwd, silu_weight_rounding, silu_weight_rounding_of)

pytestmark = pytest.mark.gpu

BOUNDARY = [31, 32, 33, 63, 64, 65, 127, 128, 129, 255, 256, 257]
N_CASES = 96


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
    # by up to 2^-8 of sum |w| |v| (tests.gpu_util.silu_weight_rounding)
    extra = silu_weight_rounding_of(b) if wl.activation == "silu" and wl.dtype == "bf16" else None
    check_forward(out, lse, ref_out, ref_lse, wl.activation, extra_tol=extra)
    check_backward(grads, oracle_bwd(b), q_off=b.q_offsets, k_off=b.kv_offsets, mags=grad_term_magnitudes_of(b))
    # rows of sequences that see no key get zero dq; keys no query sees get
    # zero dk and dv
    for s in np.nonzero(b.kv_lengths == 0)[0]:
        assert not (grads[0][int(b.q_offsets[s]):int(b.q_offsets[s + 1])] != 0).any()
    for s in np.nonzero(b.q_lengths == 0)[0]:
        for g in grads[1:]:
            assert not (g[int(b.kv_offsets[s]):int(b.kv_offsets[s + 1])] != 0).any()


LONG = [1023, 1024, 1025, 2047, 2048, 2049]


def _long_length(rng):
    kind = rng.integers(0, 7)
    if kind == 0:
        return 1
    if kind in (1, 2):
        return int(rng.choice(LONG))
    if kind == 3:
        return int(rng.integers(2, 200))
    return int(rng.integers(700, 3001))


@pytest.mark.parametrize("case", range(12))
def test_random_long_configuration(case, options):
    """Long sequences: 1 to 3 of them, up to 3000 tokens (one off 1024 and
    2048 among them), with short and single-token ones, through every
    element type, activation, mask and dQ path, against the oracle."""
    rng = np.random.default_rng(7200 + case)
    fp32 = rng.random() < 0.25
    d = int(rng.choice([32, 64, 128]))
    heads = int(rng.choice([1, 2, 4]))
    act = "silu" if rng.random() < 0.35 else "softmax"
    causal = bool(rng.random() < 0.5)
    cross = bool(rng.random() < 0.4)
    n = int(rng.integers(1, 4))
    lq = [_long_length(rng) for _ in range(n)]
    lk = [_long_length(rng) for _ in range(n)] if cross else list(lq)
    path = ["stored_ds", "recompute", "short_in_dkdv"][int(rng.integers(0, 3))]
    wl = dataclasses.replace(WORKLOADS["tiny_fp32" if fp32 else "selfattn_causal"], head_dim=d, heads=heads,
                             activation=act, causal=causal, backward=True)
    print("case %d: %s d %d heads %d %s causal %s q %s kv %s dq path %s" % (
        case, wl.dtype, d, heads, act, causal, lq, lk, path), flush=True)
    if path == "recompute":
        options("bwd_ds_store", 0)
    elif path == "short_in_dkdv":
        options("bwd_short_dq", 1)
    b = make_batch(wl, 7300 + case, q_lengths=lq, kv_lengths=lk, with_dout=True)
    dd = Dev(b)
    out, lse = dd.forward()
    grads = dd.backward(out, lse)
    torch.cuda.synchronize()
    ref_out, ref_lse = oracle_fwd(b)
    extra = silu_weight_rounding_of(b) if act == "silu" and not fp32 else None
    check_forward(out, lse, ref_out, ref_lse, act, extra_tol=extra)
    check_backward(grads, oracle_bwd(b), q_off=b.q_offsets, k_off=b.kv_offsets, mags=grad_term_magnitudes_of(b))


# ------------------------------------------------------------------ BlockAttention and pooled

def _block_config(case):
    rng = np.random.default_rng(7500 + case)
    rope = bool(rng.random() < 0.5)
    d = int(rng.choice([64, 128])) if rope else int(rng.choice([32, 64, 128]))
    fp32 = (not rope) and rng.random() < 0.2
    block = 64 if rng.random() < 0.5 else int(rng.integers(1, 65))
    heads = int(rng.choice([1, 2, 3, 4]))
    act = "silu" if rng.random() < 0.35 else "softmax"
    causal = bool(rng.random() < 0.5)
    lengths = [_length(rng) for _ in range(int(rng.integers(1, 10)))]
    base = "tiny_fp32" if fp32 else "selfattn_causal"
    wl = dataclasses.replace(WORKLOADS[base], head_dim=d, heads=heads, activation=act, causal=causal, backward=True)
    return wl, lengths, block, (10000.0 if rope else 0.0)


@pytest.mark.parametrize("case", range(24))
def test_random_block_configuration(case):
    """BlockAttention through jfa_block_forward / jfa_block_backward: block
    sizes 1 .. 64, with and without the fused rotary embedding (base 10000),
    against the oracle's block mode."""
    import math
    import oracle
    from jagged_attention_ads_amd import jfa
    from tests.gpu_util import rope_lse_bound, rope_rounding_effect
    wl, lengths, block, rope = _block_config(case)
    print("case %d: %s d %d heads %d %s causal %s block %d rope %g lengths %s" % (
        case, wl.dtype, wl.head_dim, wl.heads, wl.activation, wl.causal, block, rope, lengths), flush=True)
    b = make_batch(wl, 7600 + case, q_lengths=lengths, kv_lengths=lengths, with_dout=True)
    d = Dev(b)
    ml = max(lengths)
    out, lse = jfa.block_forward(d.q, d.k, d.v, d.qo, ml, block, d.scale, d.act, wl.causal, rope)
    grads = jfa.block_backward(d.q, d.k, d.v, out, d.do, lse, d.qo, ml, block, d.scale, d.act, wl.causal, rope)
    torch.cuda.synchronize()
    s = 1.0 / math.sqrt(wl.head_dim)
    args = (b.f64("q"), b.f64("k"), b.f64("v"))
    rb = rope if rope > 0 else None   # the oracle's "no rotary embedding" is None, the ABI's is 0
    ref_out, ref_lse = oracle.attention_fwd(*args, b.q_offsets, b.kv_offsets, s, wl.activation, wl.causal,
                                            block=block, rope_base=rb)
    lse_atol = rope_lse_bound(args[0], args[1], b.q_offsets, block, wl.causal, s) if rope else None
    # the rotary embedding: the turned Q and K are rounded to bf16 before the
    # products (tests.gpu_util.rope_rounding_effect)
    extra = rope_rounding_effect(*args, b.q_offsets, block, s, wl.activation, wl.causal, rope) if rope else None
    # SiLU: the weights of the block-token runs, over the rows the kernel
    # multiplies (turned by the rotary embedding when there is one)
    if wl.activation == "silu" and wl.dtype == "bf16":
        runs = _runs(b.q_offsets, block)
        qk = args[:2]
        if rope:
            from oracle.rope import rope as turn, sequence_positions
            qk = tuple(turn(x, sequence_positions(b.q_offsets), rope) for x in qk)
        sw = silu_weight_rounding(qk[0], qk[1], args[2], runs, runs, s, wl.causal)
        extra = sw if extra is None else extra + sw
    check_forward(out, lse, ref_out, ref_lse, wl.activation, lse_atol=lse_atol, extra_tol=extra)
    ref_g = oracle.attention_bwd(*args, b.f64("dout"), b.q_offsets, b.kv_offsets, s, wl.activation, wl.causal,
                                 block=block, rope_base=rb)
    # term magnitudes of the block-token runs (the turned rows where there is
    # a rotary embedding: the turn keeps pair lengths, not |q_c|, so those
    # cases keep the share floor alone)
    mags = None if rope else grad_term_magnitudes(*args, b.f64("dout"), _runs(b.q_offsets, block),
                                                  _runs(b.q_offsets, block), s, wl.activation, wl.causal)
    check_backward(grads, ref_g, q_off=b.q_offsets, k_off=b.kv_offsets, mags=mags)


def _runs(offsets, block):
    """Offsets of the block-token runs of every sequence, in order."""
    starts = [int(offsets[i]) + c for i in range(len(offsets) - 1)
              for c in range(0, int(offsets[i + 1] - offsets[i]), block)]
    return np.array(starts + [int(offsets[-1])], dtype=np.int64)


@pytest.mark.parametrize("case", range(16))
def test_random_pooled_configuration(case):
    """Pooled multi-head attention: 1 .. 16 seeds shared by every sequence."""
    import math
    import oracle
    from jagged_attention_ads_amd import jfa
    rng = np.random.default_rng(7800 + case)
    n_seeds = int(rng.choice([1, 2, 3, 4, 8, 16]))
    d = int(rng.choice([32, 64, 128]))
    fp32 = rng.random() < 0.2
    act = "silu" if rng.random() < 0.35 else "softmax"
    lk = [_length(rng) if rng.random() < 0.7 else int(rng.integers(300, 1500)) for _ in range(int(rng.integers(1, 9)))]
    wl = dataclasses.replace(WORKLOADS["pooled_hist"], n_seeds=n_seeds, activation=act, head_dim=d,
                             dtype="fp32" if fp32 else "bf16", heads=int(rng.choice([1, 2, 3, 8])))
    print("case %d: %s d %d heads %d %s seeds %d key lengths %s" % (
        case, wl.dtype, d, wl.heads, act, n_seeds, lk), flush=True)
    b = make_batch(wl, 7900 + case, q_lengths=[n_seeds] * len(lk), kv_lengths=lk, with_dout=True)
    dd = Dev(b)
    out, lse = jfa.pooled_forward(dd.q, dd.k, dd.v, dd.ko, dd.mk, dd.scale, act)
    grads = jfa.pooled_backward(dd.q, dd.k, dd.v, out, dd.do, lse, dd.ko, dd.mk, dd.scale, act)
    torch.cuda.synchronize()
    s = 1.0 / math.sqrt(d)
    ref_out, ref_lse = oracle.pooled_fwd(b.f64("q"), b.f64("k"), b.f64("v"), b.kv_offsets, s, act)
    extra = None
    if act == "silu" and not fp32:
        # the pooled rows: the seeds against each sequence's keys
        q_rep = np.concatenate([b.f64("q")] * len(lk), axis=0)
        extra = silu_weight_rounding(q_rep, b.f64("k"), b.f64("v"), np.arange(len(lk) + 1) * n_seeds, b.kv_offsets,
                                     s, False)
    check_forward(out, lse, ref_out, ref_lse, act, extra_tol=extra)
    ref = oracle.pooled_bwd(b.f64("q"), b.f64("k"), b.f64("v"), b.f64("dout"), b.kv_offsets, s, act)
    # term magnitudes: every sequence's seed rows, the seeds' gradient summed
    # over the sequences
    q_rep = np.concatenate([b.f64("q")] * len(lk), axis=0)
    mq, mk, mv = grad_term_magnitudes(q_rep, b.f64("k"), b.f64("v"), b.f64("dout"), np.arange(len(lk) + 1) * n_seeds,
                                      b.kv_offsets, s, act, False)
    mags = (mq.reshape(len(lk), n_seeds, *mq.shape[1:]).sum(axis=0), mk, mv)
    check_backward(grads, ref, q_off=np.array([0, n_seeds]), k_off=b.kv_offsets, mags=mags)
