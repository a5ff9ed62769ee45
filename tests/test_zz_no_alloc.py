"""The allocation-free forward (jfa_forward_noalloc: its work list in the
library's own device array) against jfa_forward with a caller workspace,
through the C ABI: bitwise equal outputs and lse, on two calls in a row per
workload, the second with a smaller batch (the array keeps the first call's
list, which the second must not reuse)."""

import pytest
import torch

from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import ORDER, make_batch
from tests.gpu_util import Dev

pytestmark = pytest.mark.gpu


@pytest.mark.parametrize("name,batches", [("selfattn_causal", (24, 5)), ("gdpa_silu", (6, 2)),
                                          ("cross_asym", (40, 7)), ("pareto_train", (200, 30)),
                                          ("tiny_fp32", (8, 3))])
def test_noalloc_forward_matches_workspace_forward(name, batches):
    for i, bsz in enumerate(batches):
        b = make_batch(name, 50 + ORDER.index(name) * 10 + i, batch=bsz)
        d = Dev(b)
        print("noalloc case: %s batch %d" % (name, bsz), flush=True)
        ref_out, ref_lse = d.forward()
        out = torch.empty_like(d.q)
        lse = torch.empty_like(ref_lse) if ref_lse is not None else None
        jfa.jfa_forward_noalloc(d.q, d.k, d.v, d.qo, d.ko, d.mq, d.mk, d.scale, d.act, d.causal, out, lse)
        torch.cuda.synchronize()
        assert torch.equal(out.view(torch.uint8), ref_out.view(torch.uint8))
        if lse is not None:
            assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))


def test_noalloc_forward_full_size():
    """The benchmark's batch, as jfa_forward's."""
    b = make_batch("selfattn_causal", 2)
    d = Dev(b)
    ref_out, ref_lse = d.forward()
    out, lse = torch.empty_like(d.q), torch.empty_like(ref_lse)
    jfa.jfa_forward_noalloc(d.q, d.k, d.v, d.qo, d.ko, d.mq, d.mk, d.scale, d.act, d.causal, out, lse)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.uint8), ref_out.view(torch.uint8))
    assert torch.equal(lse.view(torch.int32), ref_lse.view(torch.int32))
