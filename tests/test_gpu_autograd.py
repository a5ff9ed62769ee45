"""jfa.jagged_attention, the autograd wrapper: its forward is jfa.forward
(jfa.mx_forward) and its backward jfa.backward (jfa.mx_backward) with the
incoming gradient, bit for bit; inputs that need no gradient get none."""

import dataclasses

import numpy as np
import pytest
import torch

from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch
from tests.gpu_util import Dev

pytestmark = pytest.mark.gpu

CASES = [("selfattn_causal", {}), ("gdpa_silu", dict(causal=False)), ("tiny_fp32", dict(causal=True)),
         ("cross_asym", dict(heads=3))]


def _same(a, b):
    return torch.equal(a.view(torch.int16) if a.dtype == torch.bfloat16 else a,
                       b.view(torch.int16) if b.dtype == torch.bfloat16 else b)


@pytest.mark.parametrize("name,over", CASES)
def test_autograd_equals_direct_calls(name, over):
    wl = dataclasses.replace(WORKLOADS[name], backward=True, **over)
    b = make_batch(wl, 90 + [c[0] for c in CASES].index(name), batch=6, with_dout=True)
    d = Dev(b)
    q, k, v = (x.clone().requires_grad_(True) for x in (d.q, d.k, d.v))
    out = jfa.jagged_attention(q, k, v, d.qo, d.ko, d.mq, d.mk, d.scale, d.act, d.causal)
    (out.float() * d.do.float()).sum().backward()
    torch.cuda.synchronize()
    ref_out, ref_lse = d.forward()
    ref_g = d.backward(ref_out, ref_lse)
    torch.cuda.synchronize()
    assert _same(out.detach(), ref_out)
    for g, r in zip((q.grad, k.grad, v.grad), ref_g):
        assert _same(g, r)


def test_autograd_mx_equals_direct_calls():
    wl = dataclasses.replace(WORKLOADS["selfattn_causal"], backward=True)
    b = make_batch(wl, 95, batch=5, with_dout=True)
    d = Dev(b)
    q, k, v = (x.clone().requires_grad_(True) for x in (d.q, d.k, d.v))
    out = jfa.jagged_attention(q, k, v, d.qo, d.ko, d.mq, d.mk, d.scale, causal=True, mx=True)
    (out.float() * d.do.float()).sum().backward()
    torch.cuda.synchronize()
    ref_out, ref_lse = jfa.mx_forward(d.q, d.k, d.v, d.qo, d.ko, d.mq, d.mk, d.scale, True)
    ref_g = jfa.mx_backward(d.q, d.k, d.v, ref_out, d.do, ref_lse, d.qo, d.ko, d.mq, d.mk, d.scale, True)
    torch.cuda.synchronize()
    assert _same(out.detach(), ref_out)
    for g, r in zip((q.grad, k.grad, v.grad), ref_g):
        assert _same(g, r)


def test_autograd_only_requested_gradients():
    b = make_batch(dataclasses.replace(WORKLOADS["selfattn_causal"], backward=True), 96, batch=3, with_dout=True)
    d = Dev(b)
    q = d.q.clone().requires_grad_(True)
    out = jfa.jagged_attention(q, d.k, d.v, d.qo, d.ko, d.mq, d.mk, causal=True)
    out.float().sum().backward()
    torch.cuda.synchronize()
    assert q.grad is not None and torch.isfinite(q.grad.float()).all()
    assert d.k.grad is None and d.v.grad is None
    with pytest.raises(ValueError):
        jfa.jagged_attention(q, d.k, d.v, d.qo, d.ko, d.mq, d.mk, activation="silu", mx=True)


@pytest.mark.parametrize("rope", [0.0, 10000.0])
def test_autograd_block_equals_direct_calls(rope):
    wl = dataclasses.replace(WORKLOADS["selfattn_causal"], backward=True)
    lengths = [0, 1, 63, 64, 65, 130, 257]
    b = make_batch(wl, 97, q_lengths=lengths, kv_lengths=lengths, with_dout=True)
    d = Dev(b)
    q, k, v = (x.clone().requires_grad_(True) for x in (d.q, d.k, d.v))
    out = jfa.block_attention(q, k, v, d.qo, max(lengths), 64, d.scale, "softmax", True, rope)
    (out.float() * d.do.float()).sum().backward()
    torch.cuda.synchronize()
    ref_out, ref_lse = jfa.block_forward(d.q, d.k, d.v, d.qo, max(lengths), 64, d.scale, "softmax", True, rope)
    ref_g = jfa.block_backward(d.q, d.k, d.v, ref_out, d.do, ref_lse, d.qo, max(lengths), 64, d.scale, "softmax",
                               True, rope)
    torch.cuda.synchronize()
    assert _same(out.detach(), ref_out)
    for g, r in zip((q.grad, k.grad, v.grad), ref_g):
        assert _same(g, r)


@pytest.mark.parametrize("act", ["softmax", "silu"])
def test_autograd_pooled_equals_direct_calls(act):
    wl = dataclasses.replace(WORKLOADS["pooled_hist"], n_seeds=4, activation=act, heads=2)
    lk = [0, 129, 700, 1, 33]
    b = make_batch(wl, 98, q_lengths=[4] * len(lk), kv_lengths=lk, with_dout=True)
    d = Dev(b)
    s, k, v = (x.clone().requires_grad_(True) for x in (d.q, d.k, d.v))
    out = jfa.pooled_attention(s, k, v, d.ko, d.mk, d.scale, act)
    (out.float() * d.do.float()).sum().backward()
    torch.cuda.synchronize()
    ref_out, ref_lse = jfa.pooled_forward(d.q, d.k, d.v, d.ko, d.mk, d.scale, act)
    ref_g = jfa.pooled_backward(d.q, d.k, d.v, ref_out, d.do, ref_lse, d.ko, d.mk, d.scale, act)
    torch.cuda.synchronize()
    assert _same(out.detach(), ref_out)
    for g, r in zip((s.grad, k.grad, v.grad), ref_g):
        assert _same(g, r)
