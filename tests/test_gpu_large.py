"""The largest tensors the ABI accepts: just under 2^31 elements (the
documented limit), here 65 535 causal sequences of 64 tokens, 4 heads, d 128
(4.19 M tokens, 2.147e9 elements, 4.3 GB per tensor in bf16), so that byte
offsets run up to 2^32 and the MXFP8 images (32-row aligned sequences) pass 2^31
bytes: every address of the second half of the batch needs 64-bit
arithmetic.  Values are drawn on the device (seeded); sampled sequences --
the first, one in the middle and the last -- are checked against the fp64
oracle on their own, forward and backward, for the bf16 and MXFP8 paths."""

import math

import numpy as np
import pytest
import torch

import oracle
import oracle.mx as mx
from jagged_attention_ads_amd import jfa
from tests.gpu_util import check_backward, check_forward, dev, to_f64

pytestmark = pytest.mark.gpu

B, L, H, D = 65535, 64, 4, 128
SAMPLE = [0, B // 2, B - 1]


def _inputs(seed):
    g = torch.Generator(device=dev())
    g.manual_seed(seed)
    T = B * L
    q, k, v, do = (torch.randn((T, H, D), generator=g, device=dev(), dtype=torch.bfloat16) for _ in range(4))
    off = torch.arange(0, T + 1, L, dtype=torch.int32, device=dev())
    return q, k, v, do, off


def _rows(s):
    return torch.arange(s * L, (s + 1) * L, device=dev())


def _seq(x, s):
    return to_f64(x[_rows(s)])


def test_past_two_to_the_31_elements_bf16():
    q, k, v, do, off = _inputs(123)
    assert 2 ** 31 - 2 ** 16 < q.numel() < 2 ** 31 and q.numel() * 2 > 2 ** 32 - 2 ** 17
    scale = 1.0 / math.sqrt(D)
    out, lse = jfa.forward(q, k, v, off, off, L, L, scale, "softmax", True)
    dq, dk, dv = jfa.backward(q, k, v, out, do, lse, off, off, L, L, scale, "softmax", True)
    torch.cuda.synchronize()
    o1 = np.array([0, L])
    for s in SAMPLE:
        print("sequence", s, flush=True)
        qs, ks, vs, ds = (_seq(x, s) for x in (q, k, v, do))
        ref_out, ref_lse = oracle.attention_fwd(qs, ks, vs, o1, o1, scale, "softmax", True)
        check_forward(out[_rows(s)], lse[:, _rows(s)], ref_out, ref_lse, "softmax")
        ref = oracle.attention_bwd(qs, ks, vs, ds, o1, o1, scale, "softmax", True)
        check_backward((dq[_rows(s)], dk[_rows(s)], dv[_rows(s)]), ref, q_off=o1, k_off=o1)
    del q, k, v, do, out, lse, dq, dk, dv
    torch.cuda.empty_cache()


def test_past_two_to_the_31_elements_mxfp8():
    from tests.test_gpu_mx import _check as check_mx_forward
    from tests.test_gpu_mx_bwd import _check as check_mx_backward, _reference
    q, k, v, do, off = _inputs(321)
    scale = 1.0 / math.sqrt(D)
    out, lse = jfa.mx_forward(q, k, v, off, off, L, L, scale, True)
    torch.cuda.synchronize()
    o1 = np.array([0, L])
    refs = {}
    for s in SAMPLE:
        print("sequence", s, flush=True)
        qs, ks, vs = (_seq(x, s) for x in (q, k, v))
        check_mx_forward(out[_rows(s)], lse[:, _rows(s)], qs, ks, vs, o1, o1, scale, True)
        refs[s] = mx.mx_attention_fwd(qs, ks, vs, o1, o1, scale, True)
    # the backward takes the oracle's forward of the sampled sequences (out
    # rounded to bf16, lse to fp32), as tests/test_gpu_mx_bwd.py does; the
    # other sequences keep the kernel's, which changes nothing for these
    for s, (ro, rl) in refs.items():
        out[_rows(s)] = torch.from_numpy(ro.astype(np.float32)).to(dev()).to(torch.bfloat16)
        lse[:, _rows(s)] = torch.from_numpy(rl.astype(np.float32)).to(dev())
    dq, dk, dv = jfa.mx_backward(q, k, v, out, do, lse, off, off, L, L, scale, True)
    torch.cuda.synchronize()
    for s in SAMPLE:
        qs, ks, vs, ds = (_seq(x, s) for x in (q, k, v, do))
        ref, slack = _reference(qs, ks, vs, _seq(out, s), ds, lse[:, _rows(s)].double().cpu().numpy(), o1, o1,
                                scale, True)
        check_mx_backward((dq[_rows(s)], dk[_rows(s)], dv[_rows(s)]), ref, o1, o1, "sequence %d" % s, slack)
