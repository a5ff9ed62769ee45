"""C ABI checks that need no GPU: the library loads, exports every function
include/jfa.h declares, and host-side validation returns the documented
status before anything is enqueued (the pointers below are never
dereferenced: every call is rejected, or is a no-op, on the host)."""

import ctypes
import math
import os
import re

import pytest

from jagged_attention_ads_amd import jfa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "jfa.h")

OK, INVALID, UNSUPPORTED, WS_SMALL = 0, 1, 2, 3
P = 4096          # a 16-byte aligned fake device address, never dereferenced
MIS = 4098        # misaligned


def _declared():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(jfa_\w+)\s*\(", text)))


def test_header_symbols_exported():
    names = _declared()
    assert len(names) == 32, names
    L = jfa.lib()
    for n in names:
        assert hasattr(L, n), n
    assert set(names) == set(jfa.EXPORTED)


def test_status_strings():
    for code, name in jfa.STATUS_NAMES.items():
        assert jfa.jfa_status_string(code) == name
    assert "unknown" in jfa.jfa_status_string(99)


def _fwd(**kw):
    a = dict(q=P, k=P, v=P, qo=P, ko=P, batch=2, heads=2, d=64, tq=10, tk=10, mq=5, mk=5, scale=0.125,
             act=0, causal=0, dtype=0, out=P, lse=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return jfa.lib().jfa_forward(a["q"], a["k"], a["v"], a["qo"], a["ko"], a["batch"], a["heads"], a["d"], a["tq"],
                                 a["tk"], a["mq"], a["mk"], a["scale"], a["act"], a["causal"], a["dtype"],
                                 a["out"], a["lse"], a["ws"], a["wsb"], None)


def _bwd(**kw):
    a = dict(q=P, k=P, v=P, out=P, do=P, lse=P, qo=P, ko=P, batch=2, heads=2, d=64, tq=10, tk=10, mq=5, mk=5,
             scale=0.125, act=0, causal=0, dtype=0, dq=P, dk=P, dv=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return jfa.lib().jfa_backward(a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], a["qo"], a["ko"],
                                  a["batch"], a["heads"], a["d"], a["tq"], a["tk"], a["mq"], a["mk"], a["scale"],
                                  a["act"], a["causal"], a["dtype"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"],
                                  None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(qo=None), INVALID), (dict(out=None), INVALID),
    (dict(lse=None), INVALID), (dict(batch=-1), INVALID), (dict(heads=0), INVALID),
    (dict(tq=-3), INVALID), (dict(mk=-1), INVALID), (dict(scale=math.nan), INVALID),
    (dict(scale=math.inf), INVALID), (dict(scale=0.0), INVALID), (dict(scale=-0.125), INVALID),
    (dict(scale=1e-30), INVALID), (dict(scale=-math.inf), INVALID), (dict(act=2), INVALID), (dict(causal=2), INVALID), (dict(dtype=5), INVALID),
    (dict(k=MIS), INVALID), (dict(out=MIS), INVALID), (dict(tq=1 << 24, heads=2, d=128), INVALID),
    (dict(d=48), UNSUPPORTED), (dict(d=256), UNSUPPORTED), (dict(heads=257), UNSUPPORTED),
    (dict(mk=64 * 1023 + 1), UNSUPPORTED), (dict(ws=None), WS_SMALL), (dict(wsb=16), WS_SMALL),
])
def test_forward_rejects(kw, status):
    assert _fwd(**kw) == status
    assert jfa.lib().jfa_last_error()


def test_forward_noop_and_silu_without_lse():
    assert _fwd(batch=0, ws=None, wsb=0) == OK
    assert _fwd(tq=0, q=None, out=None, lse=None, ws=None, wsb=0) == OK
    # silu needs no lse; the call is still rejected here only for the workspace
    assert _fwd(act=1, lse=None, ws=None) == WS_SMALL


@pytest.mark.parametrize("kw,status", [
    (dict(do=None), INVALID), (dict(dk=None), INVALID), (dict(lse=None), INVALID), (dict(out=None), INVALID),
    (dict(dv=MIS), INVALID), (dict(mq=64 * 1023 + 1), UNSUPPORTED), (dict(d=16), UNSUPPORTED),
    (dict(wsb=100), WS_SMALL),
])
def test_backward_rejects(kw, status):
    assert _bwd(**kw) == status


def test_backward_noop_and_silu_optional():
    assert _bwd(batch=0, ws=None, wsb=0) == OK
    assert _bwd(act=1, out=None, lse=None, wsb=100) == WS_SMALL   # out/lse not required for silu


def test_workspace_sizes():
    fwd = jfa.jfa_workspace_size(256, 4, 128, 97000, 97000, 1024, 0, 0)
    bwd = jfa.jfa_workspace_size(256, 4, 128, 97000, 97000, 1024, 0, 1)
    assert 0 < fwd < bwd
    # (lse, delta) pairs [heads, total_q] fp32, then the dS store: heads x
    # (total_q // 32 + batch) block rows x ceil(max_kv_len / 32) blocks of 32 x 32 bf16
    ds = 4 * (97000 // 32 + 256) * 32 * 32 * 32 * 2
    assert bwd - fwd >= 4 * 97000 * 8 + ds
    # fp32 blocks are twice the size
    bwd32 = jfa.jfa_workspace_size(256, 4, 128, 97000, 97000, 1024, 1, 1)
    assert bwd32 - bwd >= ds
    # the forward does not depend on the key length or the element type
    assert jfa.jfa_workspace_size(256, 4, 128, 97000, 97000, 5, 1, 0) == fwd
    # for_backward = 2: the same without the dS store
    assert jfa.jfa_workspace_size(256, 4, 128, 97000, 97000, 1024, 0, 2) == bwd - ds
    assert jfa.jfa_workspace_size(256, 4, 128, 97000, 97000, 1024, 0, 3) == 0
    # a dS store beyond 16 GiB is left out (the dQ pass then recomputes dS)
    big = jfa.jfa_workspace_size(64, 64, 128, 260000, 260000, 65000, 0, 1)
    assert 0 < big < (16 << 30)
    assert big == jfa.jfa_workspace_size(64, 64, 128, 260000, 260000, 65000, 0, 2)
    assert jfa.jfa_workspace_size(2, 2, 48, 10, 10, 10, 0, 0) == 0
    assert jfa.jfa_workspace_size(2, 2, 32, 10, 10, 10, 5, 1) == 0   # bad dtype


def test_tile_shapes_and_worklist_size():
    assert jfa.jfa_tile_shape(jfa.PASS_QUERY_TILES) == (128, 64)
    assert jfa.jfa_tile_shape(jfa.PASS_KEY_TILES) == (64, 64)
    assert jfa.jfa_tile_shape(jfa.PASS_DQ_TILES) == (64, 64)
    assert jfa.jfa_tile_shape(jfa.PASS_DQ_STORED_TILES) == (256, 64)
    with pytest.raises(jfa.JfaError):
        jfa.jfa_tile_shape(7)
    # capacity bound: sum ceil(L/128) <= (T + B*127)/128 items per head
    n = jfa.jfa_worklist_bytes(jfa.PASS_QUERY_TILES, 3, 2, 300, 10)
    cap = ((300 + 3 * 127) // 128) * 2
    assert n >= 16 + 8 * cap + 4 * 4
    assert jfa.jfa_worklist_bytes(9, 3, 2, 300, 10) == 0


def test_block_offsets_validation():
    assert jfa.lib().jfa_block_offsets_count(3, 200, 64) == 200 // 64 + 3 + 1
    assert jfa.lib().jfa_block_offsets_count(3, 200, 0) == 0
    L = jfa.lib()
    assert L.jfa_block_offsets(P, 3, 200, 0, P, 100, None) == INVALID      # block < 1
    assert L.jfa_block_offsets(P, 3, 200, 64, P, 6, None) == INVALID       # out shorter than the count (7)
    assert L.jfa_block_offsets(None, 3, 200, 64, P, 7, None) == INVALID
    assert L.jfa_block_offsets(P, -1, 200, 64, P, 7, None) == INVALID


def test_forward_noalloc_rejects_sizes_beyond_its_scratch():
    """The allocation-free forward refuses, on the host and before any HIP
    call, sizes whose work list would not fit its 8 MiB device array."""
    L = jfa.lib()
    assert jfa.jfa_workspace_size(100000, 8, 128, 1000000, 1000000, 64, 0, 0) > 8 << 20
    st = L.jfa_forward_noalloc(P, P, P, P, P, 100000, 8, 128, 1000000, 1000000, 64, 64, 0.125, 0, 0, 0, P, P, None)
    assert st == UNSUPPORTED
    assert b"8 MiB" in L.jfa_last_error()
    # invalid arguments are reported as jfa_forward reports them
    st = L.jfa_forward_noalloc(P, P, P, P, P, 2, 2, 48, 10, 10, 5, 5, 0.125, 0, 0, 0, P, P, None)
    assert st == UNSUPPORTED and b"head_dim" in L.jfa_last_error()


def _blk(**kw):
    a = dict(q=P, k=P, v=P, off=P, batch=2, heads=2, d=64, total=10, max_len=5, block=64, scale=0.125, act=0,
             causal=1, dtype=0, rope=10000.0, out=P, lse=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return jfa.lib().jfa_block_forward(a["q"], a["k"], a["v"], a["off"], a["batch"], a["heads"], a["d"], a["total"],
                                       a["max_len"], a["block"], a["scale"], a["act"], a["causal"], a["dtype"],
                                       a["rope"], a["out"], a["lse"], a["ws"], a["wsb"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(block=0), INVALID), (dict(block=65), INVALID), (dict(rope=0.5), INVALID), (dict(rope=-3.0), INVALID),
    (dict(rope=math.inf), INVALID), (dict(rope=math.nan), INVALID), (dict(max_len=-1), INVALID),
    (dict(off=None), INVALID), (dict(dtype=1), UNSUPPORTED), (dict(d=32), UNSUPPORTED), (dict(q=None), INVALID),
    (dict(scale=0.0), INVALID), (dict(ws=None), WS_SMALL), (dict(wsb=64), WS_SMALL),
])
def test_block_forward_rejects(kw, status):
    """Argument checks of BlockAttention with the rotary embedding, on the
    host before anything is enqueued."""
    assert _blk(**kw) == status


def test_block_workspace_size():
    L = jfa.lib()
    assert L.jfa_block_workspace_size(4, 2, 64, 1000, 64, 0, 0) > 0
    assert L.jfa_block_workspace_size(4, 2, 64, 1000, 64, 0, 1) > L.jfa_block_workspace_size(4, 2, 64, 1000, 64, 0, 0)
    assert L.jfa_block_workspace_size(4, 2, 64, 1000, 65, 0, 0) == 0
    assert L.jfa_block_workspace_size(4, 2, 64, 1000, 64, 0, 2) == 0
    assert _blk(batch=0, ws=None, wsb=0) == OK


def _pooled(**kw):
    a = dict(seeds=P, k=P, v=P, ko=P, batch=2, n=4, heads=2, d=64, tk=10, mk=5, scale=0.125, act=0, dtype=0, out=P,
             lse=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return jfa.lib().jfa_pooled_forward(a["seeds"], a["k"], a["v"], a["ko"], a["batch"], a["n"], a["heads"], a["d"],
                                        a["tk"], a["mk"], a["scale"], a["act"], a["dtype"], a["out"], a["lse"],
                                        a["ws"], a["wsb"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(n=0), INVALID), (dict(n=257), INVALID), (dict(seeds=None), INVALID), (dict(seeds=MIS), INVALID),
    (dict(ko=None), INVALID), (dict(scale=-1.0), INVALID), (dict(d=48), UNSUPPORTED), (dict(lse=None), INVALID),
    (dict(ws=None), WS_SMALL), (dict(wsb=100), WS_SMALL), (dict(batch=1 << 24, n=200), INVALID),
])
def test_pooled_forward_rejects(kw, status):
    """Pooled attention's argument checks, on the host before anything is
    enqueued."""
    assert _pooled(**kw) == status


def test_pooled_noop_and_workspace():
    assert _pooled(batch=0, ws=None, wsb=0) == OK
    L = jfa.lib()
    assert L.jfa_pooled_workspace_size(2, 4, 2, 64, 10, 5, 0, 1) > L.jfa_pooled_workspace_size(2, 4, 2, 64, 10, 5, 0, 0) > 0
    assert L.jfa_pooled_workspace_size(2, 0, 2, 64, 10, 5, 0, 0) == 0


def _mx(**kw):
    a = dict(q=P, k=P, v=P, qo=P, ko=P, batch=2, heads=2, d=64, tq=10, tk=10, mq=5, mk=5, scale=0.125, causal=0,
             out=P, lse=P, ws=P, wsb=1 << 30)
    a.update(kw)
    return jfa.lib().jfa_mx_forward(a["q"], a["k"], a["v"], a["qo"], a["ko"], a["batch"], a["heads"], a["d"],
                                    a["tq"], a["tk"], a["mq"], a["mk"], a["scale"], a["causal"], a["out"], a["lse"],
                                    a["ws"], a["wsb"], None, None)


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(lse=None), INVALID), (dict(scale=0.0), INVALID), (dict(causal=3), INVALID),
    (dict(v=MIS), INVALID), (dict(d=32), UNSUPPORTED), (dict(d=48), UNSUPPORTED), (dict(heads=257), UNSUPPORTED),
    (dict(ws=None), WS_SMALL), (dict(wsb=100), WS_SMALL), (dict(ws=P + 16), INVALID),
])
def test_mx_forward_rejects(kw, status):
    """MXFP8 forward's argument checks, on the host before anything is
    enqueued (P is 256-byte aligned; P + 16 is not)."""
    assert _mx(**kw) == status


def test_mx_noop_and_sizes():
    assert _mx(batch=0, ws=None, wsb=0) == OK
    assert _mx(tq=0, q=None, out=None, lse=None, ws=None, wsb=0) == OK
    L = jfa.lib()
    # image: codes H * 32 (T/32 + B) * d, then the scales, each 256-aligned
    n = 100 // 32 + 3
    assert L.jfa_mx_image_bytes(3, 2, 64, 100) == 2 * 32 * n * 64 + (2 * 32 * n * 2 + 255) // 256 * 256
    assert L.jfa_mx_image_bytes(3, 2, 32, 100) == 0
    assert L.jfa_mx_workspace_size(3, 2, 64, 100, 200, 1) > L.jfa_mx_image_bytes(3, 2, 64, 100) + \
        2 * L.jfa_mx_image_bytes(3, 2, 64, 200)
    assert 0 < L.jfa_mx_workspace_size(3, 2, 64, 100, 200, 0) < L.jfa_mx_image_bytes(3, 2, 64, 100)
    assert L.jfa_mx_workspace_size(3, 2, 64, 100, 200, 2) == 0


@pytest.mark.parametrize("kw,status", [
    (dict(q=None), INVALID), (dict(q=P + 16), INVALID), (dict(d=128, heads=300), UNSUPPORTED),
    (dict(d=32), UNSUPPORTED), (dict(wsb=100), WS_SMALL), (dict(lse=None), INVALID),
])
def test_mx_attend_rejects(kw, status):
    a = dict(q=P, k=P, v=P, qo=P, ko=P, batch=2, heads=2, d=64, tq=10, tk=10, mq=5, mk=5, scale=0.125, causal=0,
             out=P, lse=P, ws=P, wsb=1 << 30)
    a.update(kw)
    assert jfa.lib().jfa_mx_attend(a["q"], a["k"], a["v"], a["qo"], a["ko"], a["batch"], a["heads"], a["d"], a["tq"],
                                   a["tk"], a["mq"], a["mk"], a["scale"], a["causal"], a["out"], a["lse"], a["ws"],
                                   a["wsb"], None, None) == status


@pytest.mark.parametrize("kw,status", [
    (dict(x=None), INVALID), (dict(off=None), INVALID), (dict(layout=2), INVALID), (dict(img=None), INVALID),
    (dict(img=P + 16), INVALID), (dict(d=128, nb=100), WS_SMALL), (dict(d=32), UNSUPPORTED), (dict(heads=0), INVALID),
])
def test_mx_quantize_rejects(kw, status):
    a = dict(x=P, off=P, batch=2, heads=2, d=64, total=10, layout=0, img=P, nb=1 << 20)
    a.update(kw)
    assert jfa.lib().jfa_mx_quantize(a["x"], a["off"], a["batch"], a["heads"], a["d"], a["total"], a["layout"],
                                     a["img"], a["nb"], None) == status


def _mxb(images=False, **kw):
    a = dict(q=P, k=P, v=P, out=P, do=P, lse=P, qo=P, ko=P, batch=2, heads=2, d=64, tq=10, tk=10, mq=5, mk=5,
             scale=0.125, causal=0, dq=P, dk=P, dv=P, ws=P, wsb=1 << 30)
    a.update(kw)
    tail = (a["qo"], a["ko"], a["batch"], a["heads"], a["d"], a["tq"], a["tk"], a["mq"], a["mk"], a["scale"],
            a["causal"], a["dq"], a["dk"], a["dv"], a["ws"], a["wsb"], None, None)
    if images:
        imgs = a.get("imgs", (ctypes.c_void_p * 7)(*([a["q"]] * 7)))
        return jfa.lib().jfa_mx_backward_images(imgs, a["out"], a["do"], a["lse"], *tail)
    return jfa.lib().jfa_mx_backward(a["q"], a["k"], a["v"], a["out"], a["do"], a["lse"], *tail)


@pytest.mark.parametrize("images", [False, True])
@pytest.mark.parametrize("kw,status", [
    (dict(lse=None), INVALID), (dict(out=None), INVALID), (dict(do=None), INVALID), (dict(dq=None), INVALID),
    (dict(dv=MIS), INVALID), (dict(scale=0.0), INVALID), (dict(causal=3), INVALID), (dict(d=32), UNSUPPORTED),
    (dict(d=96), UNSUPPORTED), (dict(heads=257), UNSUPPORTED), (dict(ws=None), WS_SMALL), (dict(wsb=100), WS_SMALL),
    (dict(mq=1 << 20), UNSUPPORTED),
])
def test_mx_backward_rejects(images, kw, status):
    """MXFP8 backward's argument checks, on the host before anything is
    enqueued, for both entry points."""
    assert _mxb(images, **kw) == status


def test_mx_backward_rejects_images_and_workspace():
    assert _mxb(False, ws=P + 16) == INVALID
    assert _mxb(True, imgs=None) == INVALID
    assert _mxb(True, imgs=(ctypes.c_void_p * 7)(*([P] * 6 + [None]))) == INVALID
    assert _mxb(True, imgs=(ctypes.c_void_p * 7)(*([P] * 6 + [P + 16]))) == INVALID
    # a side with no rows may pass NULL images and gradients
    assert _mxb(True, tk=0, dk=None, dv=None, ws=None, wsb=0, batch=0) == OK


def test_mx_backward_noop_and_sizes():
    assert _mxb(False, batch=0, ws=None, wsb=0) == OK
    assert _mxb(True, batch=0, ws=None, wsb=0) == OK
    L = jfa.lib()
    full = L.jfa_mx_backward_workspace_size(3, 2, 64, 100, 200, 1)
    lists = L.jfa_mx_backward_workspace_size(3, 2, 64, 100, 200, 0)
    # the seven images follow the lists: q, q, k, k, v, dout, dout
    assert full == lists + 4 * L.jfa_mx_image_bytes(3, 2, 64, 100) + 3 * L.jfa_mx_image_bytes(3, 2, 64, 200)
    assert lists > 2 * 2 * 100 * 4   # holds the row statistics
    assert L.jfa_mx_backward_workspace_size(3, 2, 64, 100, 200, 2) == 0
    assert L.jfa_mx_backward_workspace_size(3, 2, 48, 100, 200, 1) == 0


def test_options():
    """Path options: set, read back, reset; bad names and values rejected."""
    L = jfa.lib()
    assert [L.jfa_get_option(i) for i in range(4)] == [-1, -1, -1, -1]
    assert L.jfa_set_option(1, 0) == OK and L.jfa_get_option(1) == 0
    assert L.jfa_set_option(1, -1) == OK and L.jfa_get_option(1) == -1
    assert L.jfa_set_option(4, 0) == INVALID and L.jfa_set_option(-1, 0) == INVALID
    assert L.jfa_set_option(0, 2) == INVALID and L.jfa_set_option(0, -2) == INVALID
    assert L.jfa_get_option(4) == -2
    with jfa.option("fwd_short", False):
        assert L.jfa_get_option(3) == 0
    assert L.jfa_get_option(3) == -1
