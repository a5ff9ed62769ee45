"""MXFP8 test helpers: reading the library's MX images back into per-row
arrays (the layout include/jfa.h states), and the allowance for the decisions
the kernel takes in fp32 where the oracle's fp64 value sits on a boundary.

Test infrastructure: used by the MXFP8 tests only.
"""

import numpy as np

import oracle.mx as mx

# MXFP8 backward gates: relative L2 error of dq, dk, dv against the oracle's
# gradients rounded to bf16, per tensor and per sequence.  Kernel and oracle
# quantise the same values by the same rules; what is left is fp32 against
# fp64 arithmetic.  dP = dO.v accumulates d products in fp32 (absolute error
# about d 2^-24 times the largest term), so dS = P (dP - delta) is off by
# 1e-6 to 1e-5 of itself where dP - delta is small against dP; an E4M3
# decision of dS (or of P) within that distance of a midpoint goes the other
# way -- a few in 10^4 elements -- and moves its element by one E4M3 step
# (up to 1/8 of it).  Over a gradient that is about 1e-3 relative L2
# (measured: 3e-4 on 64-key sequences to 1.6e-3 on 1000-key ones), on top
# of bf16 roundings that fall the other way.  The plausible mistakes of a
# kernel move the gradients by 1 % or more per tensor
# (test_mx_bwd_gates_separate_mistakes).
MX_GRAD_RTOL = 5e-3
MX_GRAD_SEQ_RTOL = 1e-2


def _align256(x):
    return (x + 255) // 256 * 256


def image_parts(batch, heads, d, total):
    """(block rows N, byte offset of the scales, image bytes)."""
    n = total // 32 + batch
    rows = heads * 32 * n
    sc = _align256(rows * d)
    return n, sc, sc + _align256(rows * (d // 32))


def image_rows(offsets):
    """Image row of every packed row: 32 (off[b] / 32 + b) + i."""
    off = np.asarray(offsets, dtype=np.int64)
    out = []
    for b in range(len(off) - 1):
        out.append(32 * (off[b] // 32 + b) + np.arange(off[b + 1] - off[b]))
    return np.concatenate(out) if out else np.zeros(0, np.int64)


def decode_rows_image(img, offsets, heads, d):
    """Row image -> (codes uint8 [T, H, d], scale codes uint8 [T, H, d/32])."""
    img = np.asarray(img, dtype=np.uint8)
    off = np.asarray(offsets, dtype=np.int64)
    T = int(off[-1])
    n, sc, _ = image_parts(len(off) - 1, heads, d, T)
    codes = img[:heads * 32 * n * d].reshape(heads, 32 * n, d)
    scales = img[sc:sc + heads * 32 * n * (d // 32)].reshape(heads, 32 * n, d // 32)
    r = image_rows(off)
    return codes[:, r].transpose(1, 0, 2), scales[:, r].transpose(1, 0, 2)


def key_positions():
    """Byte of key i (0..31) within a column of a column-image block."""
    i = np.arange(32)
    return 16 * ((i // 4) % 2) + 4 * (i // 8) + i % 4


def decode_keys_image(img, offsets, heads, d):
    """Column image -> (codes uint8 [T, H, d], scale codes uint8 [T, H, d]:
    the code of the block holding each row), plus the codes of the image
    rows past each sequence's end within its last block (must be zero)."""
    img = np.asarray(img, dtype=np.uint8)
    off = np.asarray(offsets, dtype=np.int64)
    T = int(off[-1])
    n, sc, _ = image_parts(len(off) - 1, heads, d, T)
    codes = img[:heads * n * d * 32].reshape(heads, n, d, 32)
    scales = img[sc:sc + heads * n * 32 * (d // 32)].reshape(heads, n, 32, d // 32)
    pos = key_positions()
    r = image_rows(off)
    blk, i = r // 32, r % 32
    c = codes[:, blk, :, pos[i]]                 # [T, H, d] (advanced indices first)
    s = scales[:, blk].transpose(1, 0, 3, 2).reshape(len(r), heads, d)   # column 32 c + r at [r][c]
    tail = []
    for b in range(len(off) - 1):
        L = int(off[b + 1] - off[b])
        if L % 32:
            last = off[b] // 32 + b + L // 32
            tail.append(codes[:, last][..., pos[L % 32:]])
    return c, s, (np.concatenate([t.ravel() for t in tail]) if tail else np.zeros(0, np.uint8))


# E4M3 midpoints between consecutive non-negative finite values and the step there
_POS = np.sort(mx.e4m3_decode(np.arange(0x7F)))
_MID = (_POS[:-1] + _POS[1:]) / 2
_STEP = _POS[1:] - _POS[:-1]


def fwd_slack(q, k, v, q_offsets, kv_offsets, scale, causal, eps_t=1e-4, eps_e=1e-4):
    """Per-element allowance [T_q, H, d] on |out - oracle| for the weight
    quantisation's fp32 decisions near a boundary of the fp64 oracle's:
      * a block's floor when its largest visible t lies within eps_t (plus
        1e-6 |t|) of an integer: the block's weights under the other floor;
      * an element 2^(t - floor + 8) within relative eps_e of a midpoint
        between E4M3 values: one E4M3 step.
    Each changed weight dw_j adds |dw_j| |v_j| / (sum of exact weights)."""
    q = np.asarray(q, dtype=np.float64)
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    qh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(q))
    kh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(k))
    vh = np.abs(mx.mx_dequantize_keys(*mx.mx_quantize_keys(v, ko)))
    T, H, d = q.shape
    slack = np.zeros((T, H, d))
    c = scale / np.log(2.0)
    for b in range(len(qo) - 1):
        qs, qe, ks, ke = qo[b], qo[b + 1], ko[b], ko[b + 1]
        lq, lk = qe - qs, ke - ks
        if lq == 0 or lk == 0:
            continue
        vis = oracle_visible(lq, lk, causal)
        live = vis.any(axis=1)
        for h in range(H):
            t = c * (qh[qs:qe, h] @ kh[ks:ke, h].T)
            m = np.where(live, np.where(vis, t, -np.inf).max(axis=1), 0.0)
            den = np.where(live, np.where(vis, np.exp2(t - m[:, None]), 0.0).sum(axis=1), 1.0)
            dw = np.zeros((lq, lk))
            for c0 in range(0, lk, 32):
                sl = slice(c0, min(c0 + 32, lk))
                tb, vb = t[:, sl], vis[:, sl]
                bl = vb.any(axis=1)
                bmax = np.where(bl, np.where(vb, tb, -np.inf).max(axis=1), 0.0)
                f = np.floor(bmax)
                el = np.where(vb, np.exp2(tb - f[:, None] + 8), 0.0)
                w = mx.e4m3_decode(mx.e4m3_encode(el)) * np.exp2(f - 8 - m)[:, None]
                tol = eps_t + 1e-6 * np.abs(bmax)
                for alt, near in ((f - 1, bmax - f < tol), (f + 1, np.ceil(bmax) - bmax < tol)):
                    near &= bl
                    if np.any(near):
                        ela = np.where(vb, np.exp2(tb - alt[:, None] + 8), 0.0)
                        wa = mx.e4m3_decode(mx.e4m3_encode(ela)) * np.exp2(alt - 8 - m)[:, None]
                        dw[:, sl] += np.where(near[:, None], np.abs(wa - w), 0.0)
                j = np.clip(np.searchsorted(_MID, el), 1, len(_MID) - 1)
                for jj in (j - 1, j):
                    close = vb & (np.abs(el - _MID[jj]) <= eps_e * _MID[jj])
                    dw[:, sl] += np.where(close, _STEP[jj] * np.exp2(f - 8 - m)[:, None], 0.0)
            slack[qs:qe, h] = (dw @ vh[ks:ke, h]) / den[:, None]
    return slack


def oracle_visible(lq, lk, causal):
    from oracle.attention import visible_mask
    return visible_mask(lq, lk, causal)
