"""BlockAttention with fixed blocks through the C ABI (piletech.kr/articles/
112134, Detailed notes, BlockAttention item): the run offsets the device
builds, bit for bit, and forward / backward parity with the oracle's block
mode, on the unchanged q, k, v tensors."""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch, offsets_from_lengths
from tests.gpu_util import Dev, check_backward, check_forward, dev, rope_lse_bound, rope_rounding_effect

pytestmark = pytest.mark.gpu


def _runs_ref(lengths, block):
    """Run offsets as the header defines them: every sequence's runs in order,
    then the total repeated up to total // block + batch + 1 entries."""
    off = offsets_from_lengths(lengths)
    starts = [int(off[b]) + c for b, n in enumerate(lengths) for c in range(0, int(n), block)]
    count = int(off[-1]) // block + len(lengths) + 1
    return np.array(starts + [int(off[-1])] * (count - len(starts)), dtype=np.int32)


@pytest.mark.parametrize("block", [1, 7, 64])
def test_block_offsets_bit_exact(block):
    rng = np.random.default_rng(block)
    for lengths in ([0, 1, 63, 64, 65, 130, 0, 200, 5], list(rng.integers(0, 300, 2500)), [0, 0], [17]):
        off = torch.from_numpy(offsets_from_lengths(lengths).astype(np.int32)).to(dev())
        got = jfa.jfa_block_offsets(off, int(sum(lengths)), block)
        torch.cuda.synchronize()
        assert np.array_equal(got.cpu().numpy(), _runs_ref(lengths, block))
        assert np.array_equal(off.cpu().numpy(), offsets_from_lengths(lengths).astype(np.int32))


CASES = [("selfattn_causal", True), ("selfattn_causal", False), ("gdpa_silu", True)]


@pytest.mark.parametrize("name,causal", CASES)
def test_block_attention_parity(name, causal):
    wl = dataclasses.replace(WORKLOADS[name], causal=causal, backward=True)
    lengths = [0, 1, 63, 64, 65, 130, 257, 40, 128, 700]
    b = make_batch(wl, 41, q_lengths=lengths, kv_lengths=lengths, with_dout=True)
    d = Dev(b)
    T = int(b.q_offsets[-1])
    runs = jfa.jfa_block_offsets(d.qo, T, 64)
    m = min(64, max(lengths))
    out, lse = jfa.forward(d.q, d.k, d.v, runs, runs, m, m, d.scale, d.act, causal)
    grads = jfa.backward(d.q, d.k, d.v, out, d.do, lse, runs, runs, m, m, d.scale, d.act, causal)
    torch.cuda.synchronize()
    s = 1.0 / math.sqrt(wl.head_dim)
    args = (b.f64("q"), b.f64("k"), b.f64("v"))
    ref_out, ref_lse = oracle.attention_fwd(*args, b.q_offsets, b.kv_offsets, s, wl.activation, causal, block=64)
    check_forward(out, lse, ref_out, ref_lse, wl.activation)
    ref_g = oracle.attention_bwd(*args, b.f64("dout"), b.q_offsets, b.kv_offsets, s, wl.activation, causal, block=64)
    check_backward(grads, ref_g, q_off=b.q_offsets, k_off=b.kv_offsets)


def test_block_attention_full_size_sampled():
    """The benchmark's BlockAttention batch at full size: every row is
    finite, sampled sequences match the oracle."""
    b = make_batch("block_attn", 2)
    wl = b.workload
    d = Dev(b)
    T = int(b.q_offsets[-1])
    runs = jfa.jfa_block_offsets(d.qo, T, wl.block)
    m = min(wl.block, d.mq)
    out, lse = jfa.forward(d.q, d.k, d.v, runs, runs, m, m, d.scale, d.act, wl.causal)
    grads = jfa.backward(d.q, d.k, d.v, out, d.do, lse, runs, runs, m, m, d.scale, d.act, wl.causal)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and all(torch.isfinite(g).all() for g in grads)
    s = 1.0 / math.sqrt(wl.head_dim)
    for seq in (int(np.argmax(b.q_lengths)), 3, 100):
        lo, hi = int(b.q_offsets[seq]), int(b.q_offsets[seq + 1])
        one = np.array([0, hi - lo])
        sl = slice(lo, hi)
        args = (b.f64("q")[sl], b.f64("k")[sl], b.f64("v")[sl])
        ref_out, ref_lse = oracle.attention_fwd(*args, one, one, s, wl.activation, wl.causal, block=wl.block)
        check_forward(out[sl], lse[:, sl], ref_out, ref_lse, wl.activation)
        ref_g = oracle.attention_bwd(*args, b.f64("dout")[sl], one, one, s, wl.activation, wl.causal, block=wl.block)
        check_backward(tuple(g[sl] for g in grads), ref_g, q_off=one, k_off=one)


# ------------------------------------------------------------------ fused rotary embedding

ROPE_CASES = [("selfattn_causal", True, 128), ("selfattn_causal", False, 128), ("gdpa_silu", True, 128),
              ("selfattn_causal", True, 64), ("gdpa_silu", False, 64)]


@pytest.mark.parametrize("name,causal,d", ROPE_CASES)
def test_block_rope_parity(name, causal, d):
    """BlockAttention with the fused rotary embedding (base 10000) against the
    oracle (rotation of Q and K at their sequence positions, then attention
    within 64-token blocks; gradients turned back), forward and backward.
    The forward bound adds what rounding the turned Q and K to bf16 does to
    the output (tests.gpu_util.rope_rounding_effect)."""
    wl = dataclasses.replace(WORKLOADS[name], causal=causal, head_dim=d, backward=True)
    lengths = [0, 1, 63, 64, 65, 130, 257, 40, 128, 700]
    b = make_batch(wl, 61 + d, q_lengths=lengths, kv_lengths=lengths, with_dout=True)
    dv_ = Dev(b)
    print("rope case: %s causal %s d %d" % (name, causal, d), flush=True)
    out, lse = jfa.block_forward(dv_.q, dv_.k, dv_.v, dv_.qo, max(lengths), 64, dv_.scale, dv_.act, causal, 10000.0)
    grads = jfa.block_backward(dv_.q, dv_.k, dv_.v, out, dv_.do, lse, dv_.qo, max(lengths), 64, dv_.scale, dv_.act,
                               causal, 10000.0)
    torch.cuda.synchronize()
    s = 1.0 / math.sqrt(wl.head_dim)
    args = (b.f64("q"), b.f64("k"), b.f64("v"))
    ref_out, ref_lse = oracle.attention_fwd(*args, b.q_offsets, b.kv_offsets, s, wl.activation, causal, block=64,
                                            rope_base=10000.0)
    check_forward(out, lse, ref_out, ref_lse, wl.activation,
                  lse_atol=rope_lse_bound(args[0], args[1], b.q_offsets, 64, causal, s),
                  extra_tol=rope_rounding_effect(*args, b.q_offsets, 64, s, wl.activation, causal, 10000.0))
    ref_g = oracle.attention_bwd(*args, b.f64("dout"), b.q_offsets, b.kv_offsets, s, wl.activation, causal, block=64,
                                 rope_base=10000.0)
    check_backward(grads, ref_g, q_off=b.q_offsets, k_off=b.kv_offsets)


@pytest.mark.parametrize("name,causal", [("selfattn_causal", True), ("gdpa_silu", False)])
def test_block_calls_without_rope_equal_offsets_path(name, causal):
    """jfa_block_forward / jfa_block_backward with rope_base 0 are the run
    offsets plus the jagged calls, bit for bit."""
    wl = dataclasses.replace(WORKLOADS[name], causal=causal, backward=True)
    lengths = [5, 64, 130, 0, 300, 1]
    b = make_batch(wl, 71, q_lengths=lengths, kv_lengths=lengths, with_dout=True)
    d = Dev(b)
    out, lse = jfa.block_forward(d.q, d.k, d.v, d.qo, max(lengths), 64, d.scale, d.act, causal, 0.0)
    g = jfa.block_backward(d.q, d.k, d.v, out, d.do, lse, d.qo, max(lengths), 64, d.scale, d.act, causal, 0.0)
    runs = jfa.jfa_block_offsets(d.qo, int(b.q_offsets[-1]), 64)
    out2, lse2 = jfa.forward(d.q, d.k, d.v, runs, runs, 64, 64, d.scale, d.act, causal)
    g2 = jfa.backward(d.q, d.k, d.v, out2, d.do, lse2, runs, runs, 64, 64, d.scale, d.act, causal)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), out2.view(torch.uint8))
    if lse is not None:
        assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
    for x, y in zip(g, g2):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))


def test_block_rope_full_size_sampled():
    """The benchmark's BlockAttention batch with the rotary embedding: every
    row finite, sampled sequences against the oracle."""
    b = make_batch("block_attn", 2)
    wl = b.workload
    d = Dev(b)
    out, lse = jfa.block_forward(d.q, d.k, d.v, d.qo, d.mq, wl.block, d.scale, d.act, wl.causal, 10000.0)
    grads = jfa.block_backward(d.q, d.k, d.v, out, d.do, lse, d.qo, d.mq, wl.block, d.scale, d.act, wl.causal,
                               10000.0)
    torch.cuda.synchronize()
    assert torch.isfinite(out).all() and all(torch.isfinite(g).all() for g in grads)
    s = 1.0 / math.sqrt(wl.head_dim)
    for seq in (int(np.argmax(b.q_lengths)), 3, 100):
        lo, hi = int(b.q_offsets[seq]), int(b.q_offsets[seq + 1])
        one = np.array([0, hi - lo])
        sl = slice(lo, hi)
        args = (b.f64("q")[sl], b.f64("k")[sl], b.f64("v")[sl])
        ref_out, ref_lse = oracle.attention_fwd(*args, one, one, s, wl.activation, wl.causal, block=wl.block,
                                                rope_base=10000.0)
        check_forward(out[sl], lse[:, sl], ref_out, ref_lse, wl.activation,
                      lse_atol=rope_lse_bound(args[0], args[1], one, wl.block, wl.causal, s),
                      extra_tol=rope_rounding_effect(*args, one, wl.block, s, wl.activation, wl.causal, 10000.0))
        ref_g = oracle.attention_bwd(*args, b.f64("dout")[sl], one, one, s, wl.activation, wl.causal,
                                     block=wl.block, rope_base=10000.0)
        check_backward(tuple(g[sl] for g in grads), ref_g, q_off=one, k_off=one)
