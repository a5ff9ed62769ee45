"""MXFP8 test helpers: reading the library's MX images back into per-row
arrays (the layout include/jfa.h states), and the allowance for the decisions
the kernel takes in fp32 where the oracle's fp64 value sits on a boundary.

Test infrastructure: used by the MXFP8 tests only.
"""

import numpy as np

import oracle.mx as mx

# MXFP8 backward gates: relative L2 error of dq, dk, dv against the oracle's
# gradients rounded to bf16, per tensor and per sequence, once each
# element's difference is reduced by bwd_slack's allowance.  Kernel and
# oracle quantise the same values by the same rules; what is left is fp32
# (and the matrix cores' accumulation) against fp64 arithmetic.  An E4M3
# decision of P or dS within that error of a rounding midpoint, or a block
# exponent within it of a boundary, goes the other way -- a few in 10^4
# elements -- and moves its element by one E4M3 step (up to 1/8 of it).  In
# a long sequence those spread over many terms (about 1e-3 relative L2,
# below the gates without the allowance); in a short one a single flip can
# carry a gradient row (1 to 2 % measured), which the allowance takes out.
# What stays is bf16 roundings that fall the other way.  The plausible
# mistakes of a kernel move the gradients by 1 % or more per tensor, with
# the allowance taken off too (test_mx_bwd_gates_separate_mistakes).
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


def score_error(qh, kh, t, c, eps_t=1e-5, eps_sum=3e-5):
    """Bound on the kernel's error in the scores t = c q.k (log2 units) of
    one (sequence, head) block, qh [lq, d] and kh [lk, d] the dequantised
    row images: eps_t and 1e-6 |t| for fp32 evaluation, and eps_sum times
    the sum of the products' magnitudes for the block-scaled matrix cores,
    whose accumulation is not a sequence of fp32 roundings (scores 1.15e-5
    of that sum away from the oracle's were measured, 2.2e-6 in dP)."""
    return eps_t + 1e-6 * np.abs(t) + c * eps_sum * (np.abs(qh) @ np.abs(kh).T)


def fwd_slack(q, k, v, q_offsets, kv_offsets, scale, causal, eps_t=1e-5, eps_sum=3e-5):
    """Per-element allowance [T_q, H, d] on |out - oracle| for the weight
    quantisation's decisions, which the kernel takes on scores known to
    score_error's bound dt: each weight, under every block floor its block's
    largest score can take within dt of the oracle's, and at both ends of
    its own score's interval (E4M3 rounding is monotone), differs from the
    oracle's weight by at most the largest of those changes, dw_j.  Each
    adds |dw_j| |v_j| / (sum of exact weights) to the output."""
    q = np.asarray(q, dtype=np.float64)
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    qh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(q))
    kh = mx.mx_dequantize_rows(*mx.mx_quantize_rows(k))
    vh = np.abs(mx.mx_dequantize_keys(*mx.mx_quantize_keys(v, ko)))
    T, H, d = q.shape
    slack = np.zeros((T, H, d))
    c = scale / np.log(2.0)

    def wq(tt, f, m):   # quantised weight of scores tt under block floor f (saturating at 448)
        return mx.e4m3_decode(mx.e4m3_encode(np.minimum(np.exp2(tt - f[:, None] + 8), mx.E4M3_MAX))) * \
            np.exp2(f - 8 - m)[:, None]

    for b in range(len(qo) - 1):
        qs, qe, ks, ke = qo[b], qo[b + 1], ko[b], ko[b + 1]
        lq, lk = qe - qs, ke - ks
        if lq == 0 or lk == 0:
            continue
        vis = oracle_visible(lq, lk, causal)
        live = vis.any(axis=1)
        for h in range(H):
            t = c * (qh[qs:qe, h] @ kh[ks:ke, h].T)
            dt = score_error(qh[qs:qe, h], kh[ks:ke, h], t, c, eps_t, eps_sum)
            m = np.where(live, np.where(vis, t, -np.inf).max(axis=1), 0.0)
            den = np.where(live, np.where(vis, np.exp2(t - m[:, None]), 0.0).sum(axis=1), 1.0)
            dw = np.zeros((lq, lk))
            for c0 in range(0, lk, 32):
                sl = slice(c0, min(c0 + 32, lk))
                tb, vb, db = t[:, sl], vis[:, sl], dt[:, sl]
                bl = vb.any(axis=1)
                top = lambda x: np.where(bl, np.where(vb, x, -np.inf).max(axis=1), 0.0)   # noqa: E731
                f = np.floor(top(tb))
                f_lo, f_hi = np.floor(top(tb - db)), np.floor(top(tb + db))
                cur = wq(tb, f, m)
                best = np.zeros_like(tb)
                for dlt in range(int((f_lo - f).min(initial=0)), int((f_hi - f).max(initial=0)) + 1):
                    fa = f + dlt
                    ok = ((fa >= f_lo) & (fa <= f_hi))[:, None]
                    ch = np.maximum(np.abs(wq(tb + db, fa, m) - cur), np.abs(wq(tb - db, fa, m) - cur))
                    best = np.maximum(best, np.where(ok, ch, 0.0))
                dw[:, sl] = np.where(vb, best, 0.0)
            slack[qs:qe, h] = (dw @ vh[ks:ke, h]) / den[:, None]
    return slack


def oracle_visible(lq, lk, causal):
    from oracle.attention import visible_mask
    return visible_mask(lq, lk, causal)


def _q(m, sc):
    """Dequantised E4M3 value of magnitudes m under block scale sc (values
    past 448 sc cannot occur under that scale and are taken at 448 sc)."""
    return mx.e4m3_decode(mx.e4m3_encode(np.minimum(m / sc, mx.E4M3_MAX))) * sc


def _flip_allowance(x, rel, axis):
    """Per-element bound on |Q(x') - Q(x)| over every x' with |x' - x| <=
    rel |x| elementwise, Q being the oracle's mx_quantize_matrix (blocks of
    32 along `axis` of the 2-D x, fitted exponent; rel an array like x, or a
    scalar).  E4M3 rounding is monotone, so under one block exponent the
    largest change of an element is at an end of its interval; the block's
    exponent is the fitted one of its largest magnitude, which lies between
    the largest lower and the largest upper end, and every exponent in that
    range is tried."""
    x = np.asarray(x, dtype=np.float64)
    rel = np.broadcast_to(np.asarray(rel, dtype=np.float64), x.shape)
    y, r = (x, rel) if axis == 0 else (x.T, rel.T)
    out = np.zeros_like(y)
    for r0 in range(0, y.shape[0], 32):
        mag, rb = np.abs(y[r0:r0 + 32]), r[r0:r0 + 32]
        lo, hi = mag * np.maximum(1 - rb, 0.0), mag * (1 + rb)
        ex = mx.e8m0_exponent_fit(mag.max(axis=0))
        ex_lo, ex_hi = mx.e8m0_exponent_fit(lo.max(axis=0)), mx.e8m0_exponent_fit(hi.max(axis=0))
        cur = _q(mag, np.exp2(ex.astype(np.float64))[None])
        a = np.zeros_like(mag)
        for dlt in range(int((ex_lo - ex).min(initial=0)), int((ex_hi - ex).max(initial=0)) + 1):
            alt = ex + dlt
            ok = ((alt >= ex_lo) & (alt <= ex_hi))[None]
            sa = np.exp2(alt.astype(np.float64))[None]
            step = np.maximum(np.abs(_q(hi, sa) - cur), np.abs(_q(lo, sa) - cur))
            a = np.maximum(a, np.where(ok, step, 0.0))
        out[r0:r0 + 32] = a
    return out if axis == 0 else out.T


def bwd_slack(q, k, v, out, dout, lse, q_offsets, kv_offsets, scale, causal, eps_p=1e-6, eps_sum=3e-5):
    """Per-element allowances (dq, dk, dv), each like its gradient, on
    |gradient - oracle| for the E4M3 decisions of P and dS that the kernel
    takes in fp32 where the fp64 oracle's value sits within the kernel's
    error of a rounding midpoint or of a block exponent's boundary.  The
    block-scaled products' sums (S = Q K^T and dP = dO V^T over d terms) are
    taken as known to eps_sum times the sum of the terms' magnitudes (the
    matrix cores' accumulation is not a sequence of fp32 roundings: a
    weight 1.7e-5 below the oracle's, from a score off by 1.4e-4 against
    terms summing to about 64, and forward scores 1.15e-5 of that sum
    away, were measured), the exponential and lse to
    eps_p: P to eps_p + scale eps_sum sum|q||k| relative, dS = P (dP -
    delta) to that plus eps_sum (sum|dO||v| + sum|dO||O|) / |dP - delta|.
    Each possible change dx of a quantised operand element adds |dx| times
    the magnitude of the other operand to the gradient elements it feeds: P
    to dV along queries with dO's column image, dS to dK along queries with
    Q's, dS to dQ along keys with K's."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    rows = lambda x: mx.mx_dequantize_rows(*mx.mx_quantize_rows(x))       # noqa: E731
    cols = lambda x, o: mx.mx_dequantize_keys(*mx.mx_quantize_keys(x, o))  # noqa: E731
    q_r, k_r, v_r, do_r = rows(q), rows(k), rows(v), rows(dout)
    q_c, do_c, k_c = np.abs(cols(q, qo)), np.abs(cols(dout, qo)), np.abs(cols(k, ko))
    delta = (dout * out).sum(axis=2)
    mag_delta = np.abs(dout * out).sum(axis=2)
    aq, ak, av = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(qo) - 1):
        qs, qe, ks, ke = int(qo[b]), int(qo[b + 1]), int(ko[b]), int(ko[b + 1])
        lq, lk = qe - qs, ke - ks
        if lq == 0 or lk == 0:
            continue
        vis = oracle_visible(lq, lk, causal)
        for h in range(q.shape[1]):
            lrow = lse[h, qs:qe]
            ok = vis & np.isfinite(lrow)[:, None]
            s = scale * (q_r[qs:qe, h] @ k_r[ks:ke, h].T)
            p = np.where(ok, np.exp(s - np.where(np.isfinite(lrow), lrow, 0.0)[:, None]), 0.0)
            rel_p = eps_p + scale * eps_sum * (np.abs(q_r[qs:qe, h]) @ np.abs(k_r[ks:ke, h]).T)
            dp = do_r[qs:qe, h] @ v_r[ks:ke, h].T
            mdp = np.abs(do_r[qs:qe, h]) @ np.abs(v_r[ks:ke, h]).T
            dd = dp - delta[qs:qe, h][:, None]
            ds = p * dd
            with np.errstate(divide="ignore", invalid="ignore"):
                rel_ds = rel_p + eps_sum * (mdp + mag_delta[qs:qe, h][:, None]) / np.abs(dd)
            rel_ds = np.where(np.isfinite(rel_ds), rel_ds, 1.0)
            av[ks:ke, h] = _flip_allowance(p, rel_p, 0).T @ do_c[qs:qe, h]
            ak[ks:ke, h] = scale * (_flip_allowance(ds, rel_ds, 0).T @ q_c[qs:qe, h])
            aq[qs:qe, h] = scale * (_flip_allowance(ds, rel_ds, 1) @ k_c[ks:ke, h])
    return aq, ak, av
