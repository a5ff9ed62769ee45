"""Bit-exact bookkeeping of the HIP path.

* the device-built work lists equal the oracle's CPU enumeration bit for bit;
* offsets are left unchanged;
* every (row, head) slot of out / lse / dq / dk / dv is written, and nothing
  beyond the tensors (guard rows) is;
* outputs are bitwise reproducible, bitwise invariant (up to the permutation)
  under reordering of the sequences, and a sequence's outputs do not depend on
  its neighbours (no leakage, even from neighbours holding +-1e4).
"""

import dataclasses
import functools
import math

import numpy as np
import pytest
import torch

import oracle
from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import WORKLOADS, draw_lengths, make_batch, offsets_from_lengths
from tests.gpu_util import Dev, dev, values_to_device

pytestmark = pytest.mark.gpu


def _worklist_case(name, batch, causal):
    """Offsets drawn from the workload's length laws (no values: the lists
    depend on the offsets alone)."""
    wl = WORKLOADS[name]
    rng = np.random.default_rng(7)
    lq = draw_lengths(rng, wl.q_law, batch)
    lk = lq.copy() if wl.kv_law is None else draw_lengths(rng, wl.kv_law, batch)
    return offsets_from_lengths(lq), offsets_from_lengths(lk), wl.heads, causal


WL_CASES = [
    ("selfattn_causal", 64, True),
    ("selfattn_causal", 64, False),
    ("cross_asym", 512, False),
    ("cross_asym", 300, True),
    ("pareto_train", 1024, True),
    ("gdpa_silu", 256, True),
    # more sequences than a builder workgroup has threads (chunked scans)
    ("cross_asym", 3000, False),
    ("selfattn_causal", 2500, True),
    # more sequences than the builder stages in LDS (8191): offsets read from
    # global memory
    ("selfattn_causal", 9000, True),
    ("pareto_train", 12000, False),
]


@functools.lru_cache(maxsize=None)
def _worklist_ref(name, batch, causal, pass_):
    """The oracle's list for a case, as int32 [n, 2] (computed once for both bodies)."""
    qo, ko, H, causal = _worklist_case(name, batch, causal)
    tile, block = jfa.jfa_tile_shape(pass_)
    if pass_ != jfa.PASS_KEY_TILES:
        costs = oracle.fwd_tile_costs(qo, ko, tile, block, causal)
    else:
        costs = oracle.kv_tile_costs(qo, ko, block, tile, causal)
    ref = oracle.worklist(costs, H)
    return np.array([[b, (t << 8) | h] for b, h, t, _ in ref], dtype=np.int32).reshape(-1, 2)


@pytest.mark.parametrize("name,batch,causal", WL_CASES)
@pytest.mark.parametrize("pass_", [jfa.PASS_QUERY_TILES, jfa.PASS_KEY_TILES, jfa.PASS_DQ_TILES,
                                   jfa.PASS_DQ_STORED_TILES])
def test_worklist_bit_exact(name, batch, causal, pass_):
    qo, ko, H, causal = _worklist_case(name, batch, causal)
    tile = jfa.jfa_tile_shape(pass_)[0]
    ref_arr = _worklist_ref(name, batch, causal, pass_)
    qo_d = torch.from_numpy(qo.astype(np.int32)).to(dev())
    ko_d = torch.from_numpy(ko.astype(np.int32)).to(dev())
    lq, lk = np.diff(qo), np.diff(ko)
    items, tile_start, records = jfa.build_worklist(pass_, qo_d, ko_d, H, int(qo[-1]), int(ko[-1]), int(lq.max()),
                                                    int(lk.max()), causal, with_records=True)
    assert np.array_equal(items.numpy(), ref_arr)
    # the kernels' per-item records: offsets, lengths, head, tile and sequence of each
    # item in list order, then lq = -1 up to the capacity
    n = len(ref_arr)
    bb = ref_arr[:, 0].astype(np.int64)
    want = np.stack([qo[bb], lq[bb], ko[bb], lk[bb], ref_arr[:, 1] & 255, ref_arr[:, 1] >> 8,
                     bb, np.zeros(n, np.int64)], axis=1).astype(np.int32)
    rec = records.numpy()
    assert np.array_equal(rec[:n], want)
    assert np.all(rec[n:, 1] == -1)
    lens = lk if pass_ == jfa.PASS_KEY_TILES else lq
    assert np.array_equal(tile_start.numpy(), offsets_from_lengths(-(-lens // tile)).astype(np.int32))
    # offsets untouched
    assert np.array_equal(qo_d.cpu().numpy(), qo.astype(np.int32))
    assert np.array_equal(ko_d.cpu().numpy(), ko.astype(np.int32))


def _bits(t):
    return t.contiguous().view(torch.int16 if t.element_size() == 2 else torch.int32).cpu().numpy()


@pytest.mark.parametrize("name", ["selfattn_causal", "gdpa_silu", "tiny_fp32"])
def test_every_slot_written_once_and_guards_intact(name):
    wl = dataclasses.replace(WORKLOADS[name], backward=True)
    b = make_batch(wl, 3, q_lengths=[5, 0, 140, 64, 1], kv_lengths=[5, 7, 140, 0, 1] if not wl.causal
                   else [5, 0, 140, 64, 1], with_dout=True)
    d = Dev(b)
    G = 3   # guard rows after each tensor
    T_q, H, D = d.q.shape
    T_k = d.k.shape[0]
    canary = float("nan")

    def buf(rows):
        return torch.full((rows + G, H, D), canary, dtype=d.q.dtype, device=dev())

    out_b, dq_b, dk_b, dv_b = buf(T_q), buf(T_q), buf(T_k), buf(T_k)
    lse_b = torch.full((H * T_q + 7,), canary, dtype=torch.float32, device=dev())
    out, dq, dk, dv = out_b[:T_q], dq_b[:T_q], dk_b[:T_k], dv_b[:T_k]
    lse = lse_b[:H * T_q].view(H, T_q) if wl.activation == "softmax" else None
    ws = jfa.workspace(len(b.q_lengths), H, D, T_q, T_k, d.mk, d.q.dtype, True, dev())
    jfa.jfa_forward(d.q, d.k, d.v, d.qo, d.ko, d.mq, d.mk, d.scale, d.act, d.causal, out, lse, ws)
    jfa.jfa_backward(d.q, d.k, d.v, out, d.do, lse, d.qo, d.ko, d.mq, d.mk, d.scale, d.act, d.causal, dq, dk, dv, ws)
    torch.cuda.synchronize()
    for t in (out, dq, dk, dv):
        assert not torch.isnan(t).any(), "a slot was left unwritten"
    for t, n in ((out_b, T_q), (dq_b, T_q), (dk_b, T_k), (dv_b, T_k)):
        assert torch.isnan(t[n:]).all(), "a guard row was written"
    if lse is not None:
        assert not torch.isnan(lse).any()
        assert torch.isnan(lse_b[H * T_q:]).all()
    else:
        assert torch.isnan(lse_b).all()


@pytest.mark.parametrize("name", ["selfattn_causal", "gdpa_silu", "pareto_train"])
def test_bitwise_reproducible(name):
    b = make_batch(name, 5, batch=48 if name != "pareto_train" else 256)
    d = Dev(b)
    runs = []
    for _ in range(2):
        out, lse = d.forward()
        g = d.backward(out, lse)
        torch.cuda.synchronize()
        runs.append([_bits(x) for x in (out,) + tuple(g)] + ([lse.cpu().numpy()] if lse is not None else []))
    for a, z in zip(*runs):
        assert np.array_equal(a, z)


@pytest.mark.parametrize("name", ["selfattn_causal", "cross_asym", "gdpa_silu"])
def test_permutation_bitwise(name):
    wl = dataclasses.replace(WORKLOADS[name], backward=True)
    b = make_batch(wl, 9, batch=20, with_dout=True)
    perm = np.random.default_rng(1).permutation(20)
    qo, ko = b.q_offsets, b.kv_offsets

    def cat(x, o):
        return np.concatenate([x[o[p]:o[p + 1]] for p in perm])
    b2 = dataclasses.replace(b, q_lengths=b.q_lengths[perm], kv_lengths=b.kv_lengths[perm],
                             q_offsets=offsets_from_lengths(b.q_lengths[perm]),
                             kv_offsets=offsets_from_lengths(b.kv_lengths[perm]),
                             q=cat(b.q, qo), k=cat(b.k, ko), v=cat(b.v, ko), dout=cat(b.dout, qo))
    res = []
    for bb in (b, b2):
        d = Dev(bb)
        out, lse = d.forward()
        g = d.backward(out, lse)
        torch.cuda.synchronize()
        res.append((out, lse, g))
    (o1, l1, g1), (o2, l2, g2) = res
    assert np.array_equal(cat(_bits(o1), qo), _bits(o2))
    if l1 is not None:
        assert np.array_equal(np.concatenate([l1.cpu().numpy()[:, qo[p]:qo[p + 1]] for p in perm], axis=1),
                              l2.cpu().numpy())
    assert np.array_equal(cat(_bits(g1[0]), qo), _bits(g2[0]))
    assert np.array_equal(cat(_bits(g1[1]), ko), _bits(g2[1]))
    assert np.array_equal(cat(_bits(g1[2]), ko), _bits(g2[2]))


@pytest.mark.parametrize("causal", [False, True])
def test_no_leakage_from_extreme_neighbours(causal):
    """A 77-token sequence between neighbours holding +-1e4 (and a last
    sequence that ends exactly at the end of the allocation) gives bitwise the
    same outputs as the sequence alone."""
    wl = dataclasses.replace(WORKLOADS["selfattn_causal"], causal=causal, head_dim=64)
    lens = [130, 77, 200]
    b = make_batch(wl, 11, q_lengths=lens, kv_lengths=lens, with_dout=True)
    big = np.float32(1e4)
    rng = np.random.default_rng(2)
    for name in ("q", "k", "v", "dout"):
        arr = getattr(b, name)
        for s in (0, 2):
            o = b.q_offsets
            sl = slice(o[s], o[s + 1])
            signs = np.where(rng.random(arr[sl].shape) < 0.5, -big, big).astype(np.float32)
            arr[sl] = (signs.view(np.uint32) >> 16).astype(np.uint16)
    alone = make_batch(wl, 11, q_lengths=[77], kv_lengths=[77], with_dout=True)
    o = b.q_offsets
    for name in ("q", "k", "v", "dout"):
        setattr(alone, name, getattr(b, name)[o[1]:o[2]].copy())
    res = []
    for bb in (b, alone):
        d = Dev(bb)
        out, lse = d.forward()
        g = d.backward(out, lse)
        torch.cuda.synchronize()
        res.append((out, lse, g))
    (o1, l1, g1), (o2, l2, g2) = res
    r = slice(o[1], o[2])
    assert np.array_equal(_bits(o1[r]), _bits(o2))
    assert np.array_equal(l1[:, r].cpu().numpy(), l2.cpu().numpy())
    for x, y in zip(g1, g2):
        assert np.array_equal(_bits(x[r]), _bits(y))
    assert torch.isfinite(o2).all()


def test_noop_and_zero_rows():
    H, D = 2, 64
    q = torch.zeros((0, H, D), dtype=torch.bfloat16, device=dev())
    qo = torch.zeros(1, dtype=torch.int32, device=dev())
    out, lse = jfa.forward(q, q, q, qo, qo, 0, 0)
    assert out.shape == (0, H, D)
    # keys nobody reads: dk = dv = 0
    qo = torch.tensor([0, 0], dtype=torch.int32, device=dev())
    ko = torch.tensor([0, 5], dtype=torch.int32, device=dev())
    k = torch.randn((5, H, D), device=dev()).to(torch.bfloat16)
    dq, dk, dv = jfa.backward(q, k, k, q, q, torch.empty((H, 0), device=dev()), qo, ko, 0, 5)
    torch.cuda.synchronize()
    assert (dk == 0).all() and (dv == 0).all()


# malformed offsets, each breaking one rule of the offsets contract, for
# q lengths [5, 0, 4] (total 9, longest 5); the call is made with the valid
# totals and maxima (the last case lowers max_q_len / max_kv_len instead)
_BAD_OFFSETS = {
    "first_not_zero": ([1, 5, 5, 9], 5, "first offset not 0"),
    "decreasing": ([0, 5, 4, 9], 5, "offsets decrease"),
    "last_not_total": ([0, 5, 5, 8], 5, "last offset differs from the total"),
    "too_long": ([0, 5, 5, 9], 4, "a length exceeds the maximum"),
}


@pytest.mark.parametrize("case", ["valid"] + sorted(_BAD_OFFSETS))
def test_device_offsets_check(case, options):
    """The offsets check on: malformed offsets are rejected on the device, no
    output is written and jfa_check_device_error names the rule; valid ones
    run as usual and report JFA_OK."""
    options("check_offsets", 1)
    H, D, T, B = 2, 64, 9, 3
    qo_list, mx, words = ([0, 5, 5, 9], 5, None) if case == "valid" else _BAD_OFFSETS[case]
    g = torch.Generator().manual_seed(7)
    q, k, v, do = (torch.randn((T, H, D), generator=g).to(torch.bfloat16).to(dev()) for _ in range(4))
    qo = torch.tensor(qo_list, dtype=torch.int32, device=dev())
    nan = float("nan")
    out = torch.full((T, H, D), nan, dtype=torch.bfloat16, device=dev())
    lse = torch.full((H, T), nan, dtype=torch.float32, device=dev())
    dq, dk, dv = (torch.full((T, H, D), nan, dtype=torch.bfloat16, device=dev()) for _ in range(3))
    ws_f = jfa.workspace(B, H, D, T, T, mx, q.dtype, 0, dev())
    ws_b = jfa.workspace(B, H, D, T, T, mx, q.dtype, 1, dev())
    jfa.jfa_forward(q, k, v, qo, qo, mx, mx, 0.125, "softmax", True, out, lse, ws_f)
    st_f, msg_f = jfa.jfa_check_device_error(ws_f)
    if case == "valid":
        jfa.jfa_backward(q, k, v, out, do, lse, qo, qo, mx, mx, 0.125, "softmax", True, dq, dk, dv, ws_b)
        st_b, _ = jfa.jfa_check_device_error(ws_b)
        assert st_f == 0 and st_b == 0
        for t in (out, lse, dq, dk, dv):
            assert torch.isfinite(t).all()
        return
    # the backward gets the forward's untouched outputs (NaN): nothing runs on them
    jfa.jfa_backward(q, k, v, out, do, lse, qo, qo, mx, mx, 0.125, "softmax", True, dq, dk, dv, ws_b)
    st_b, msg_b = jfa.jfa_check_device_error(ws_b)
    assert st_f == 1 and st_b == 1   # JFA_ERR_INVALID_ARGUMENT
    assert words in msg_f and words in msg_b
    for t in (out, lse, dq, dk, dv):
        assert torch.isnan(t).all(), "an output was written from rejected offsets"
    # offsets untouched
    assert qo.cpu().tolist() == qo_list


def test_device_offsets_check_keyless(options):
    """Rejected offsets in a batch of short sequences, one of them without
    keys: the dQ launch, which there only zeroes the rows of sequences
    without keys, writes nothing either."""
    options("check_offsets", 1)
    H, D, T, B = 2, 64, 9, 3
    g = torch.Generator().manual_seed(8)
    q, k, v, do = (torch.randn((T, H, D), generator=g).to(torch.bfloat16).to(dev()) for _ in range(4))
    qo = torch.tensor([1, 5, 5, 9], dtype=torch.int32, device=dev())   # first offset not 0
    ko = torch.tensor([0, 0, 4, 9], dtype=torch.int32, device=dev())   # sequence 0 has no keys
    out = torch.zeros((T, H, D), dtype=torch.bfloat16, device=dev())
    lse = torch.zeros((H, T), dtype=torch.float32, device=dev())
    nan = float("nan")
    dq, dk, dv = (torch.full((T, H, D), nan, dtype=torch.bfloat16, device=dev()) for _ in range(3))
    ws_b = jfa.workspace(B, H, D, T, T, 5, q.dtype, 1, dev())
    jfa.jfa_backward(q, k, v, out, do, lse, qo, ko, 5, 5, 0.125, "softmax", True, dq, dk, dv, ws_b)
    st, msg = jfa.jfa_check_device_error(ws_b)
    assert st == 1 and "first offset not 0" in msg
    for t in (dq, dk, dv):
        assert torch.isnan(t).all(), "an output was written from rejected offsets"


@pytest.mark.parametrize("recompute", [False, True])
def test_no_keys_at_all(recompute, options):
    """total_kv = 0 with queries present: only the query-tile list is built and
    the row statistics run as a kernel of their own; out = 0, lse = -inf and
    dq = 0 for every row (both dQ passes)."""
    if recompute:
        options("bwd_ds_store", 0)
    H, D = 2, 128
    q = torch.randn((7, H, D), device=dev()).to(torch.bfloat16)
    do = torch.randn((7, H, D), device=dev()).to(torch.bfloat16)
    k = torch.zeros((0, H, D), dtype=torch.bfloat16, device=dev())
    qo = torch.tensor([0, 3, 7], dtype=torch.int32, device=dev())
    ko = torch.zeros(3, dtype=torch.int32, device=dev())
    for causal in (False, True):
        out, lse = jfa.forward(q, k, k, qo, ko, 4, 0, causal=causal)
        dq, dk, dv = jfa.backward(q, k, k, out, do, lse, qo, ko, 4, 0, causal=causal)
        torch.cuda.synchronize()
        assert (out == 0).all() and (dq == 0).all()
        assert torch.isneginf(lse).all()
        assert dk.shape == (0, H, D) and dv.shape == (0, H, D)


def test_profiled_calls_with_partial_events():
    """jfa_forward_profiled / jfa_backward_profiled record only the non-NULL
    entries of their events array (the timed steps of the benchmark keep two
    of them), and give the plain calls' results bit for bit."""
    import ctypes
    import importlib.util
    import os
    spec = importlib.util.spec_from_file_location(
        "bench", os.path.join(os.path.dirname(os.path.dirname(os.path.abspath(__file__))), "bench.py"))
    bench = importlib.util.module_from_spec(spec)
    spec.loader.exec_module(bench)
    b = make_batch("selfattn_causal", 5, batch=6)
    d = Dev(b)
    out, lse = d.forward()
    grads = d.backward(out, lse)
    T_q, H, D = d.q.shape
    B = len(b.q_lengths)
    L = jfa.lib()
    P = lambda t: ctypes.c_void_p(t.data_ptr())  # noqa: E731
    stream = ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)
    ev = bench.HipEvents()
    pair = ev.create(2)
    fe = (ctypes.c_void_p * 3)()
    fe[1], fe[2] = pair[0], pair[1]
    be = (ctypes.c_void_p * 5)()
    be[2], be[3] = pair[0], pair[1]
    out2, lse2 = torch.empty_like(out), torch.empty_like(lse)
    dq2, dk2, dv2 = (torch.empty_like(g) for g in grads)
    ws_f = jfa.workspace(B, H, D, T_q, d.k.shape[0], d.mk, d.q.dtype, 0, d.q.device)
    ws_b = jfa.workspace(B, H, D, T_q, d.k.shape[0], d.mk, d.q.dtype, 1, d.q.device)
    st = L.jfa_forward_profiled(P(d.q), P(d.k), P(d.v), P(d.qo), P(d.ko), B, H, D, T_q, d.k.shape[0], d.mq, d.mk,
                                d.scale, 0, 1, 0, P(out2), P(lse2), P(ws_f), ws_f.numel(), stream,
                                ctypes.cast(fe, ctypes.c_void_p))
    assert st == 0
    torch.cuda.synchronize()
    assert ev.ms(pair[0], pair[1]) > 0
    st = L.jfa_backward_profiled(P(d.q), P(d.k), P(d.v), P(out2), P(d.do), P(lse2), P(d.qo), P(d.ko), B, H, D, T_q,
                                 d.k.shape[0], d.mq, d.mk, d.scale, 0, 1, 0, P(dq2), P(dk2), P(dv2), P(ws_b),
                                 ws_b.numel(), stream, ctypes.cast(be, ctypes.c_void_p))
    assert st == 0
    torch.cuda.synchronize()
    assert ev.ms(pair[0], pair[1]) > 0
    ev.destroy(pair)
    for x, y in zip((out, lse) + tuple(grads), (out2, lse2, dq2, dk2, dv2)):
        assert torch.equal(x.view(torch.uint8), y.view(torch.uint8))
