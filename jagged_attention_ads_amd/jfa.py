"""Thin Python binding of libjfa.so (argument marshalling only).

The functions named like the C entry points (jfa_forward, jfa_backward, ...)
take torch tensors, check their dtype/device/contiguity, pass raw device
pointers and the current HIP stream, and raise JfaError on a non-zero
status.  Every step of the computation runs in the library's HIP kernels;
torch only provides device memory and the stream.  ``forward`` and
``backward`` additionally allocate the outputs and the workspace.

There is no fallback: without the built library (see
``jagged_attention_ads_amd.build``) every call raises.
"""

import ctypes
import math
import os

import torch

_LIB_PATH = os.path.join(os.path.dirname(os.path.abspath(__file__)), "libjfa.so")

JFA_OK = 0
STATUS_NAMES = {0: "JFA_OK", 1: "JFA_ERR_INVALID_ARGUMENT", 2: "JFA_ERR_UNSUPPORTED",
                3: "JFA_ERR_WORKSPACE_TOO_SMALL", 4: "JFA_ERR_HIP"}
ACTIVATIONS = {"softmax": 0, "silu": 1}
DTYPES = {torch.bfloat16: 0, torch.float32: 1}
PASS_QUERY_TILES = 0
PASS_KEY_TILES = 1
PASS_DQ_TILES = 2
PASS_DQ_STORED_TILES = 3

EXPORTED = ("jfa_workspace_size", "jfa_forward", "jfa_backward", "jfa_forward_profiled", "jfa_backward_profiled",
            "jfa_worklist_bytes", "jfa_tile_shape", "jfa_build_worklist", "jfa_check_device_error",
            "jfa_block_offsets_count", "jfa_block_offsets", "jfa_status_string", "jfa_last_error",
            "jfa_forward_noalloc", "jfa_bbs_batch_count", "jfa_bbs_plan", "jfa_block_workspace_size",
            "jfa_block_forward", "jfa_block_backward", "jfa_pooled_workspace_size", "jfa_pooled_forward",
            "jfa_pooled_backward", "jfa_mx_image_bytes", "jfa_mx_quantize", "jfa_mx_workspace_size",
            "jfa_mx_forward", "jfa_mx_attend", "jfa_mx_backward_workspace_size", "jfa_mx_backward",
            "jfa_mx_backward_images", "jfa_set_option", "jfa_get_option")
MX_LAYOUTS = {"rows": 0, "keys": 1, "columns": 1}
OPTIONS = {"check_offsets": 0, "bwd_ds_store": 1, "bwd_short_dq": 2, "fwd_short": 3}
BBS_COSTS = {"tokens": 0, "pairs": 1}


class JfaError(RuntimeError):
    def __init__(self, status, message=""):
        self.status = status
        super().__init__("%s: %s" % (STATUS_NAMES.get(status, str(status)), message))


_lib = None

_i32, _sz, _vp, _f32 = ctypes.c_int32, ctypes.c_size_t, ctypes.c_void_p, ctypes.c_float


def lib():
    """The loaded libjfa.so (loaded on first use; raises if it was never built)."""
    global _lib
    if _lib is None:
        if not os.path.exists(_LIB_PATH):
            raise ImportError("libjfa.so is not built at %s; run `python -m jagged_attention_ads_amd.build`"
                              % _LIB_PATH)
        L = ctypes.CDLL(_LIB_PATH)
        L.jfa_workspace_size.restype = _sz
        L.jfa_workspace_size.argtypes = [_i32] * 8
        L.jfa_forward.restype = ctypes.c_int
        L.jfa_forward.argtypes = [_vp, _vp, _vp, _vp, _vp] + [_i32] * 7 + [_f32, _i32, _i32, _i32, _vp, _vp, _vp, _sz, _vp]
        L.jfa_forward_noalloc.restype = ctypes.c_int
        L.jfa_forward_noalloc.argtypes = [_vp, _vp, _vp, _vp, _vp] + [_i32] * 7 + [_f32, _i32, _i32, _i32, _vp, _vp,
                                                                            _vp]
        L.jfa_backward.restype = ctypes.c_int
        L.jfa_backward.argtypes = [_vp] * 8 + [_i32] * 7 + [_f32, _i32, _i32, _i32, _vp, _vp, _vp, _vp, _sz, _vp]
        L.jfa_forward_profiled.restype = ctypes.c_int
        L.jfa_forward_profiled.argtypes = L.jfa_forward.argtypes + [_vp]
        L.jfa_backward_profiled.restype = ctypes.c_int
        L.jfa_backward_profiled.argtypes = L.jfa_backward.argtypes + [_vp]
        L.jfa_worklist_bytes.restype = _sz
        L.jfa_worklist_bytes.argtypes = [_i32] * 5
        L.jfa_tile_shape.restype = ctypes.c_int
        L.jfa_tile_shape.argtypes = [_i32, ctypes.POINTER(_i32), ctypes.POINTER(_i32)]
        L.jfa_build_worklist.restype = ctypes.c_int
        L.jfa_build_worklist.argtypes = [_i32, _vp, _vp] + [_i32] * 7 + [_vp, _sz, _vp]
        L.jfa_block_offsets_count.restype = ctypes.c_int64
        L.jfa_block_offsets_count.argtypes = [_i32, _i32, _i32]
        L.jfa_block_offsets.restype = ctypes.c_int
        L.jfa_block_offsets.argtypes = [_vp, _i32, _i32, _i32, _vp, ctypes.c_int64, _vp]
        L.jfa_check_device_error.restype = ctypes.c_int
        L.jfa_check_device_error.argtypes = [_vp, _vp]
        L.jfa_status_string.restype = ctypes.c_char_p
        L.jfa_status_string.argtypes = [ctypes.c_int]
        L.jfa_bbs_batch_count.restype = ctypes.c_int64
        L.jfa_bbs_batch_count.argtypes = [ctypes.c_int64, _i32]
        L.jfa_bbs_plan.restype = ctypes.c_int
        L.jfa_bbs_plan.argtypes = [_vp, ctypes.c_int64, _i32, _i32, _vp, _vp]
        L.jfa_block_workspace_size.restype = _sz
        L.jfa_block_workspace_size.argtypes = [_i32] * 7
        L.jfa_block_forward.restype = ctypes.c_int
        L.jfa_block_forward.argtypes = [_vp] * 4 + [_i32] * 6 + [_f32, _i32, _i32, _i32, _f32, _vp, _vp, _vp, _sz,
                                                                 _vp, _vp]
        L.jfa_block_backward.restype = ctypes.c_int
        L.jfa_block_backward.argtypes = [_vp] * 7 + [_i32] * 6 + [_f32, _i32, _i32, _i32, _f32] + [_vp] * 4 + [
            _sz, _vp, _vp]
        L.jfa_pooled_workspace_size.restype = _sz
        L.jfa_pooled_workspace_size.argtypes = [_i32] * 8
        L.jfa_pooled_forward.restype = ctypes.c_int
        L.jfa_pooled_forward.argtypes = [_vp] * 4 + [_i32] * 6 + [_f32, _i32, _i32, _vp, _vp, _vp, _sz, _vp, _vp]
        L.jfa_pooled_backward.restype = ctypes.c_int
        L.jfa_pooled_backward.argtypes = [_vp] * 7 + [_i32] * 6 + [_f32, _i32, _i32] + [_vp] * 4 + [_sz, _vp, _vp]
        L.jfa_mx_image_bytes.restype = _sz
        L.jfa_mx_image_bytes.argtypes = [_i32] * 4
        L.jfa_mx_quantize.restype = ctypes.c_int
        L.jfa_mx_quantize.argtypes = [_vp, _vp] + [_i32] * 5 + [_vp, _sz, _vp]
        L.jfa_mx_workspace_size.restype = _sz
        L.jfa_mx_workspace_size.argtypes = [_i32] * 6
        L.jfa_mx_forward.restype = ctypes.c_int
        L.jfa_mx_forward.argtypes = [_vp] * 5 + [_i32] * 7 + [_f32, _i32, _vp, _vp, _vp, _sz, _vp, _vp]
        L.jfa_mx_attend.restype = ctypes.c_int
        L.jfa_mx_attend.argtypes = L.jfa_mx_forward.argtypes
        L.jfa_set_option.restype = ctypes.c_int
        L.jfa_set_option.argtypes = [_i32, _i32]
        L.jfa_get_option.restype = ctypes.c_int32
        L.jfa_get_option.argtypes = [_i32]
        L.jfa_mx_backward_workspace_size.restype = _sz
        L.jfa_mx_backward_workspace_size.argtypes = [_i32] * 6
        L.jfa_mx_backward.restype = ctypes.c_int
        L.jfa_mx_backward.argtypes = [_vp] * 8 + [_i32] * 7 + [_f32, _i32] + [_vp] * 4 + [_sz, _vp, _vp]
        L.jfa_mx_backward_images.restype = ctypes.c_int
        L.jfa_mx_backward_images.argtypes = [_vp] * 6 + [_i32] * 7 + [_f32, _i32] + [_vp] * 4 + [_sz, _vp, _vp]
        L.jfa_last_error.restype = ctypes.c_char_p
        L.jfa_last_error.argtypes = []
        _lib = L
    return _lib


def _check(status):
    if status != JFA_OK:
        raise JfaError(status, lib().jfa_last_error().decode())


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _dtype_code(t):
    if t.dtype not in DTYPES:
        raise TypeError("values must be bfloat16 or float32, got %s" % t.dtype)
    return DTYPES[t.dtype]


def _values(name, t, dtype):
    if not t.is_cuda or not t.is_contiguous() or t.dim() != 3 or t.dtype != dtype:
        raise ValueError("%s must be a contiguous 3-D %s CUDA tensor [rows, heads, head_dim]" % (name, dtype))


def _offsets(name, t):
    if not t.is_cuda or t.dtype != torch.int32 or t.dim() != 1 or not t.is_contiguous():
        raise ValueError("%s must be a contiguous 1-D int32 CUDA tensor" % name)


# ---------------------------------------------------------------- C names

def jfa_status_string(status):
    return lib().jfa_status_string(status).decode()


def jfa_workspace_size(batch, heads, head_dim, total_q, total_kv, max_kv_len, dtype, for_backward):
    """dtype: a torch dtype (bfloat16 / float32) or its jfa_dtype code."""
    code = DTYPES[dtype] if isinstance(dtype, torch.dtype) else int(dtype)
    return lib().jfa_workspace_size(batch, heads, head_dim, total_q, total_kv, int(max_kv_len), code,
                                    int(for_backward))


def jfa_worklist_bytes(pass_, batch, heads, total_q, total_kv):
    return lib().jfa_worklist_bytes(pass_, batch, heads, total_q, total_kv)


def jfa_tile_shape(pass_):
    a, b = _i32(), _i32()
    _check(lib().jfa_tile_shape(pass_, ctypes.byref(a), ctypes.byref(b)))
    return a.value, b.value


def jfa_forward(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, activation, causal, out, lse,
                workspace):
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _values(name, t, q.dtype)
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    T_q, H, D = q.shape
    _check(lib().jfa_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets), q_offsets.numel() - 1,
                             H, D, T_q, k.shape[0], int(max_q_len), int(max_kv_len), float(scale),
                             ACTIVATIONS[activation], int(bool(causal)), dt, _ptr(out), _ptr(lse), _ptr(workspace),
                             workspace.numel() if workspace is not None else 0, _stream()))


def jfa_forward_noalloc(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, activation, causal, out,
                        lse):
    """jfa_forward without a workspace: the library's own device scratch holds the work list."""
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out)):
        _values(name, t, q.dtype)
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    T_q, H, D = q.shape
    _check(lib().jfa_forward_noalloc(_ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets),
                                     q_offsets.numel() - 1, H, D, T_q, k.shape[0], int(max_q_len), int(max_kv_len),
                                     float(scale), ACTIVATIONS[activation], int(bool(causal)), dt, _ptr(out),
                                     _ptr(lse), _stream()))


def jfa_backward(q, k, v, out, dout, lse, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, activation, causal,
                 dq, dk, dv, workspace):
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout), ("dq", dq), ("dk", dk), ("dv", dv)):
        _values(name, t, q.dtype)
    if out is not None:
        _values("out", out, q.dtype)
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    T_q, H, D = q.shape
    _check(lib().jfa_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(q_offsets),
                              _ptr(kv_offsets), q_offsets.numel() - 1, H, D, T_q, k.shape[0], int(max_q_len),
                              int(max_kv_len), float(scale), ACTIVATIONS[activation], int(bool(causal)), dt,
                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(workspace),
                              workspace.numel() if workspace is not None else 0, _stream()))


def jfa_build_worklist(pass_, q_offsets, kv_offsets, heads, total_q, total_kv, max_q_len, max_kv_len, causal,
                       out):
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    _check(lib().jfa_build_worklist(pass_, _ptr(q_offsets), _ptr(kv_offsets), q_offsets.numel() - 1, heads,
                                    total_q, total_kv, int(max_q_len), int(max_kv_len), int(bool(causal)),
                                    _ptr(out), out.numel(), _stream()))


def jfa_block_offsets(offsets, total, block=64):
    """Device int32 offsets of the `block`-token runs of every sequence,
    padded with empty sequences to jfa_block_offsets_count entries (see
    include/jfa.h).  Use them as both q and kv offsets, with batch
    len(result) - 1, for block attention."""
    _offsets("offsets", offsets)
    batch = offsets.numel() - 1
    n = lib().jfa_block_offsets_count(batch, int(total), int(block))
    out = torch.empty(max(n, 1), dtype=torch.int32, device=offsets.device)
    _check(lib().jfa_block_offsets(_ptr(offsets), batch, int(total), int(block), _ptr(out), out.numel(), _stream()))
    return out


def jfa_check_device_error(workspace):
    """Synchronises the current stream; returns (status, message) of the
    offsets check of the last call that built a work list in `workspace`
    (with the offsets check on)."""
    st = lib().jfa_check_device_error(_ptr(workspace), _stream())
    return st, (lib().jfa_last_error().decode() if st != JFA_OK else "")


def jfa_bbs_plan(lengths, base_batch=128, cost="tokens"):
    """Base Batch Shuffling over host lengths (a sequence of ints or an int32
    numpy array).  Returns (perm, batch_start) as int64 numpy arrays: merged
    batch i is perm[batch_start[i]:batch_start[i+1]]."""
    import numpy as np
    lens = np.ascontiguousarray(lengths, dtype=np.int32)
    n = int(lens.size)
    nb = lib().jfa_bbs_batch_count(n, int(base_batch))
    perm = np.empty(max(n, 1), dtype=np.int64)
    start = np.empty(nb + 1, dtype=np.int64)
    _check(lib().jfa_bbs_plan(lens.ctypes.data if n else None, n, int(base_batch), BBS_COSTS[cost],
                              perm.ctypes.data if n else None, start.ctypes.data))
    return perm[:n], start


def block_forward(q, k, v, offsets, max_len, block=64, scale=None, activation="softmax", causal=True,
                  rope_base=0.0):
    """BlockAttention (with the fused rotary embedding when rope_base > 0)
    over the sequences of `offsets`; returns (out, lse)."""
    _offsets("offsets", offsets)
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _values(name, t, q.dtype)
    T, H, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    B = offsets.numel() - 1
    out = torch.empty_like(q)
    lse = torch.empty((H, T), dtype=torch.float32, device=q.device) if activation == "softmax" else None
    ws = torch.empty(max(lib().jfa_block_workspace_size(B, H, D, T, block, dt, 0), 1), dtype=torch.uint8,
                     device=q.device)
    _check(lib().jfa_block_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(offsets), B, H, D, T, int(max_len), int(block),
                                   float(scale), ACTIVATIONS[activation], int(bool(causal)), dt, float(rope_base),
                                   _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(), None))
    return out, lse


def block_backward(q, k, v, out, dout, lse, offsets, max_len, block=64, scale=None, activation="softmax",
                   causal=True, rope_base=0.0):
    """Gradients (dq, dk, dv) of block_forward."""
    _offsets("offsets", offsets)
    dt = _dtype_code(q)
    for name, t in (("q", q), ("k", k), ("v", v), ("dout", dout)):
        _values(name, t, q.dtype)
    T, H, D = q.shape
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    B = offsets.numel() - 1
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(lib().jfa_block_workspace_size(B, H, D, T, block, dt, 1), 1), dtype=torch.uint8,
                     device=q.device)
    _check(lib().jfa_block_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(offsets), B,
                                    H, D, T, int(max_len), int(block), float(scale), ACTIVATIONS[activation],
                                    int(bool(causal)), dt, float(rope_base), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                    ws.numel(), _stream(), None))
    return dq, dk, dv


def pooled_forward(seeds, k, v, kv_offsets, max_kv_len, scale=None, activation="softmax"):
    """Pooled multi-head attention: seeds [n, H, d] shared by every sequence
    of kv_offsets; returns (out [batch * n, H, d], lse or None)."""
    _offsets("kv_offsets", kv_offsets)
    dt = _dtype_code(seeds)
    for name, t in (("seeds", seeds), ("k", k), ("v", v)):
        _values(name, t, seeds.dtype)
    n, H, D = seeds.shape
    B = kv_offsets.numel() - 1
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = torch.empty((B * n, H, D), dtype=seeds.dtype, device=seeds.device)
    lse = torch.empty((H, B * n), dtype=torch.float32, device=seeds.device) if activation == "softmax" else None
    ws = torch.empty(max(lib().jfa_pooled_workspace_size(B, n, H, D, k.shape[0], int(max_kv_len), dt, 0), 1),
                     dtype=torch.uint8, device=seeds.device)
    _check(lib().jfa_pooled_forward(_ptr(seeds), _ptr(k), _ptr(v), _ptr(kv_offsets), B, n, H, D, k.shape[0],
                                    int(max_kv_len), float(scale), ACTIVATIONS[activation], dt, _ptr(out), _ptr(lse),
                                    _ptr(ws), ws.numel(), _stream(), None))
    return out, lse


def pooled_backward(seeds, k, v, out, dout, lse, kv_offsets, max_kv_len, scale=None, activation="softmax"):
    """Gradients (dseeds, dk, dv) of pooled_forward."""
    _offsets("kv_offsets", kv_offsets)
    dt = _dtype_code(seeds)
    n, H, D = seeds.shape
    B = kv_offsets.numel() - 1
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dseeds, dk, dv = torch.empty_like(seeds), torch.empty_like(k), torch.empty_like(v)
    ws = torch.empty(max(lib().jfa_pooled_workspace_size(B, n, H, D, k.shape[0], int(max_kv_len), dt, 1), 1),
                     dtype=torch.uint8, device=seeds.device)
    _check(lib().jfa_pooled_backward(_ptr(seeds), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse),
                                     _ptr(kv_offsets), B, n, H, D, k.shape[0], int(max_kv_len), float(scale),
                                     ACTIVATIONS[activation], dt, _ptr(dseeds), _ptr(dk), _ptr(dv), _ptr(ws),
                                     ws.numel(), _stream(), None))
    return dseeds, dk, dv


def set_option(name, value):
    """Sets a process-wide path option (see jfa.h): value None (the library's
    choice), False / 0 or True / 1.  Returns the previous value (None, 0 or
    1)."""
    old = lib().jfa_get_option(OPTIONS[name])
    v = -1 if value is None else int(bool(value))
    _check(lib().jfa_set_option(OPTIONS[name], v))
    return None if old < 0 else old


class option:
    """Context manager: a path option set for the duration of a block."""

    def __init__(self, name, value):
        self.name, self.value = name, value

    def __enter__(self):
        self.old = set_option(self.name, self.value)
        return self

    def __exit__(self, *exc):
        set_option(self.name, self.old)
        return False


def mx_quantize(x, offsets, layout):
    """MX image of a bf16 tensor x [total, H, d] (layout "rows" for q and k,
    "keys" = "columns" for v; the backward also takes q, k and dout as
    "columns") as a uint8 device tensor; see jfa.h for its layout."""
    _offsets("offsets", offsets)
    _values("x", x, torch.bfloat16)
    T, H, D = x.shape
    B = offsets.numel() - 1
    n = lib().jfa_mx_image_bytes(B, H, D, T)
    img = torch.zeros(max(n, 1), dtype=torch.uint8, device=x.device)
    _check(lib().jfa_mx_quantize(_ptr(x), _ptr(offsets), B, H, D, T, MX_LAYOUTS[layout], _ptr(img), img.numel(),
                                 _stream()))
    return img


def mx_forward(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale=None, causal=False, ws=None,
               events=None):
    """MXFP8 softmax attention forward (bf16 in and out); returns (out, lse)."""
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    for name, t in (("q", q), ("k", k), ("v", v)):
        _values(name, t, torch.bfloat16)
    T_q, H, D = q.shape
    B = q_offsets.numel() - 1
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    out = torch.empty_like(q)
    lse = torch.empty((H, T_q), dtype=torch.float32, device=q.device)
    if ws is None:
        ws = torch.empty(max(lib().jfa_mx_workspace_size(B, H, D, T_q, k.shape[0], 1), 1), dtype=torch.uint8,
                         device=q.device)
    _check(lib().jfa_mx_forward(_ptr(q), _ptr(k), _ptr(v), _ptr(q_offsets), _ptr(kv_offsets), B, H, D, T_q,
                                k.shape[0], int(max_q_len), int(max_kv_len), float(scale), int(bool(causal)),
                                _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(), events))
    return out, lse


def mx_attend(q_image, k_image, v_image, q_offsets, kv_offsets, heads, head_dim, total_q, total_kv, max_q_len,
              max_kv_len, scale=None, causal=False, device=None, events=None):
    """MXFP8 attention from MX images (mx_quantize's output: q and k "rows",
    v "keys"); returns (out bf16 [total_q, heads, head_dim], lse)."""
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    B = q_offsets.numel() - 1
    dev_ = q_image.device if device is None else device
    scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
    out = torch.empty((total_q, heads, head_dim), dtype=torch.bfloat16, device=dev_)
    lse = torch.empty((heads, total_q), dtype=torch.float32, device=dev_)
    ws = torch.empty(max(lib().jfa_mx_workspace_size(B, heads, head_dim, total_q, total_kv, 0), 1),
                     dtype=torch.uint8, device=dev_)
    _check(lib().jfa_mx_attend(_ptr(q_image), _ptr(k_image), _ptr(v_image), _ptr(q_offsets), _ptr(kv_offsets), B,
                               heads, head_dim, total_q, total_kv, int(max_q_len), int(max_kv_len), float(scale),
                               int(bool(causal)), _ptr(out), _ptr(lse), _ptr(ws), ws.numel(), _stream(), events))
    return out, lse


MX_BACKWARD_IMAGES = (("q", "rows"), ("q", "columns"), ("k", "rows"), ("k", "columns"), ("v", "rows"),
                      ("dout", "rows"), ("dout", "columns"))


def mx_backward(q, k, v, out, dout, lse, q_offsets, kv_offsets, max_q_len, max_kv_len, scale=None, causal=False,
                ws=None, events=None):
    """MXFP8 softmax attention backward from bf16 tensors (the library
    quantises the seven operand images); returns (dq, dk, dv) in bf16."""
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    for name, t in (("q", q), ("k", k), ("v", v), ("out", out), ("dout", dout)):
        _values(name, t, torch.bfloat16)
    T_q, H, D = q.shape
    B = q_offsets.numel() - 1
    scale = 1.0 / math.sqrt(D) if scale is None else scale
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if ws is None:
        ws = torch.empty(max(lib().jfa_mx_backward_workspace_size(B, H, D, T_q, k.shape[0], 1), 1),
                         dtype=torch.uint8, device=q.device)
    _check(lib().jfa_mx_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(out), _ptr(dout), _ptr(lse), _ptr(q_offsets),
                                 _ptr(kv_offsets), B, H, D, T_q, k.shape[0], int(max_q_len), int(max_kv_len),
                                 float(scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                 ws.numel(), _stream(), events))
    return dq, dk, dv


def mx_backward_images(images, out, dout, lse, q_offsets, kv_offsets, heads, head_dim, total_q, total_kv,
                       max_q_len, max_kv_len, scale=None, causal=False, ws=None, events=None):
    """MXFP8 backward from the seven MX images, in the order of
    MX_BACKWARD_IMAGES (mx_quantize's output); out and dout (bf16) give
    delta.  Returns (dq, dk, dv) in bf16."""
    _offsets("q_offsets", q_offsets)
    _offsets("kv_offsets", kv_offsets)
    if len(images) != len(MX_BACKWARD_IMAGES):
        raise ValueError("mx_backward_images takes %d images" % len(MX_BACKWARD_IMAGES))
    B = q_offsets.numel() - 1
    dev_ = out.device
    scale = 1.0 / math.sqrt(head_dim) if scale is None else scale
    dq = torch.empty((total_q, heads, head_dim), dtype=torch.bfloat16, device=dev_)
    dk = torch.empty((total_kv, heads, head_dim), dtype=torch.bfloat16, device=dev_)
    dv = torch.empty_like(dk)
    if ws is None:
        ws = torch.empty(max(lib().jfa_mx_backward_workspace_size(B, heads, head_dim, total_q, total_kv, 0), 1),
                         dtype=torch.uint8, device=dev_)
    ptrs = (ctypes.c_void_p * len(images))(*[_ptr(x) for x in images])
    _check(lib().jfa_mx_backward_images(ptrs, _ptr(out), _ptr(dout), _ptr(lse), _ptr(q_offsets), _ptr(kv_offsets), B,
                                        heads, head_dim, total_q, total_kv, int(max_q_len), int(max_kv_len),
                                        float(scale), int(bool(causal)), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(ws),
                                        ws.numel(), _stream(), events))
    return dq, dk, dv


# ---------------------------------------------------------------- allocating wrappers

def workspace(batch, heads, head_dim, total_q, total_kv, max_kv_len, dtype, for_backward, device):
    n = jfa_workspace_size(batch, heads, head_dim, total_q, total_kv, max_kv_len, dtype, for_backward)
    return torch.empty(max(n, 1), dtype=torch.uint8, device=device)


def forward(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale=None, activation="softmax",
            causal=False, ws=None):
    """Returns (out, lse); lse is None for silu."""
    T_q, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    out = torch.empty_like(q)
    lse = torch.empty((H, T_q), dtype=torch.float32, device=q.device) if activation == "softmax" else None
    if ws is None:
        ws = workspace(q_offsets.numel() - 1, H, D, T_q, k.shape[0], max_kv_len, q.dtype, False, q.device)
    jfa_forward(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, activation, causal, out, lse, ws)
    return out, lse


def backward(q, k, v, out, dout, lse, q_offsets, kv_offsets, max_q_len, max_kv_len, scale=None,
             activation="softmax", causal=False, ws=None):
    """Returns (dq, dk, dv)."""
    T_q, H, D = q.shape
    if scale is None:
        scale = 1.0 / math.sqrt(D)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    if ws is None:
        ws = workspace(q_offsets.numel() - 1, H, D, T_q, k.shape[0], max_kv_len, q.dtype, True, q.device)
    jfa_backward(q, k, v, out, dout, lse, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, activation,
                 causal, dq, dk, dv, ws)
    return dq, dk, dv


def build_worklist(pass_, q_offsets, kv_offsets, heads, total_q, total_kv, max_q_len, max_kv_len, causal,
                   with_records=False):
    """Runs the device work-list builder; returns (items int32 [n, 2], tile_start int32 [B+1]) on the host.

    with_records: also return the per-item records the attention kernels read,
    int32 [capacity, 8] = (q start, q length, kv start, kv length, head, tile, sequence, 0),
    q length -1 past the item count (an internal layout, for tests)."""
    B = q_offsets.numel() - 1
    nbytes = jfa_worklist_bytes(pass_, B, heads, total_q, total_kv)
    buf = torch.zeros(max(nbytes, 16), dtype=torch.uint8, device=q_offsets.device)
    jfa_build_worklist(pass_, q_offsets, kv_offsets, heads, total_q, total_kv, max_q_len, max_kv_len, causal, buf)
    host = buf.cpu()
    words = host.view(torch.int32)
    count = int(words[0])
    tile = jfa_tile_shape(pass_)[0]
    rows = total_kv if pass_ == PASS_KEY_TILES else total_q
    cap = ((rows + B * (tile - 1)) // tile) * heads
    items = words[4:4 + 2 * cap].view(cap, 2)[:count].clone()
    tile_start = words[4 + 2 * cap:4 + 2 * cap + B + 1].clone()
    if not with_records:
        return items, tile_start
    meta_off = (16 + 8 * cap + 4 * (B + 1) + 31) // 32 * 32
    records = words[meta_off // 4:meta_off // 4 + 8 * cap].view(cap, 8).clone()
    return items, tile_start, records


# ---------------------------------------------------------------- autograd

class _JaggedAttention(torch.autograd.Function):
    """forward: jfa_forward (or the MXFP8 path); backward: jfa_backward with
    the saved out and lse.  Only marshalling: both passes run in the
    library's kernels."""

    @staticmethod
    def forward(ctx, q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, activation, causal, mx):
        if mx:
            out, lse = mx_forward(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, causal)
        else:
            out, lse = forward(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale, activation, causal)
        ctx.save_for_backward(q, k, v, out, q_offsets, kv_offsets, *(() if lse is None else (lse,)))
        ctx.args = (max_q_len, max_kv_len, scale, activation, causal, mx)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, q_offsets, kv_offsets, *rest = ctx.saved_tensors
        lse = rest[0] if rest else None
        max_q_len, max_kv_len, scale, activation, causal, mx = ctx.args
        dout = dout.contiguous()
        if mx:
            dq, dk, dv = mx_backward(q, k, v, out, dout, lse, q_offsets, kv_offsets, max_q_len, max_kv_len, scale,
                                     causal)
        else:
            dq, dk, dv = backward(q, k, v, out, dout, lse, q_offsets, kv_offsets, max_q_len, max_kv_len, scale,
                                  activation, causal)
        need = ctx.needs_input_grad
        return (dq if need[0] else None, dk if need[1] else None, dv if need[2] else None,
                None, None, None, None, None, None, None, None)


def jagged_attention(q, k, v, q_offsets, kv_offsets, max_q_len, max_kv_len, scale=None, activation="softmax",
                     causal=False, mx=False):
    """Jagged attention as a differentiable PyTorch op: out [T_q, H, d] from
    q [T_q, H, d], k and v [T_kv, H, d] and int32 offsets [B + 1] (device
    tensors, contiguous; bf16 or fp32, MXFP8 from bf16 with mx=True, softmax
    only).  The backward runs jfa_backward (or jfa_mx_backward) with the
    saved output and lse."""
    D = q.shape[-1]
    scale = 1.0 / math.sqrt(D) if scale is None else float(scale)
    if mx and activation != "softmax":
        raise ValueError("the MXFP8 path is softmax attention")
    return _JaggedAttention.apply(q, k, v, q_offsets, kv_offsets, int(max_q_len), int(max_kv_len), scale,
                                  activation, bool(causal), bool(mx))


class _BlockAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, q, k, v, offsets, max_len, block, scale, activation, causal, rope_base):
        out, lse = block_forward(q, k, v, offsets, max_len, block, scale, activation, causal, rope_base)
        ctx.save_for_backward(q, k, v, out, offsets, *(() if lse is None else (lse,)))
        ctx.args = (max_len, block, scale, activation, causal, rope_base)
        return out

    @staticmethod
    def backward(ctx, dout):
        q, k, v, out, offsets, *rest = ctx.saved_tensors
        max_len, block, scale, activation, causal, rope_base = ctx.args
        dq, dk, dv = block_backward(q, k, v, out, dout.contiguous(), rest[0] if rest else None, offsets, max_len,
                                    block, scale, activation, causal, rope_base)
        need = ctx.needs_input_grad
        return (dq if need[0] else None, dk if need[1] else None, dv if need[2] else None,
                None, None, None, None, None, None, None)


def block_attention(q, k, v, offsets, max_len, block=64, scale=None, activation="softmax", causal=True,
                    rope_base=0.0):
    """BlockAttention (jfa_block_forward / jfa_block_backward) as a
    differentiable PyTorch op; rope_base > 0 fuses the rotary embedding."""
    scale = 1.0 / math.sqrt(q.shape[-1]) if scale is None else float(scale)
    return _BlockAttention.apply(q, k, v, offsets, int(max_len), int(block), scale, activation, bool(causal),
                                 float(rope_base))


class _PooledAttention(torch.autograd.Function):
    @staticmethod
    def forward(ctx, seeds, k, v, kv_offsets, max_kv_len, scale, activation):
        out, lse = pooled_forward(seeds, k, v, kv_offsets, max_kv_len, scale, activation)
        ctx.save_for_backward(seeds, k, v, out, kv_offsets, *(() if lse is None else (lse,)))
        ctx.args = (max_kv_len, scale, activation)
        return out

    @staticmethod
    def backward(ctx, dout):
        seeds, k, v, out, kv_offsets, *rest = ctx.saved_tensors
        max_kv_len, scale, activation = ctx.args
        ds, dk, dv = pooled_backward(seeds, k, v, out, dout.contiguous(), rest[0] if rest else None, kv_offsets,
                                     max_kv_len, scale, activation)
        need = ctx.needs_input_grad
        return (ds if need[0] else None, dk if need[1] else None, dv if need[2] else None, None, None, None, None)


def pooled_attention(seeds, k, v, kv_offsets, max_kv_len, scale=None, activation="softmax"):
    """Pooled multi-head attention (jfa_pooled_forward / jfa_pooled_backward)
    as a differentiable PyTorch op: out [batch * n_seeds, H, d]."""
    scale = 1.0 / math.sqrt(seeds.shape[-1]) if scale is None else float(scale)
    return _PooledAttention.apply(seeds, k, v, kv_offsets, int(max_kv_len), scale, activation)
