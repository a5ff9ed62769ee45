"""MXFP8 jagged attention forward: OCP Microscaling E4M3 operands, fp64.

TEST INFRASTRUCTURE ONLY (see the package docstring for the rule and for the
citation keys used below).

[GEM-MFU, Key points: MXFP8] and [GEM-MFU, Detailed notes: MXFP8 item]: the
model trains in MXFP8, a microscaled 8-bit format; the attention's softmax
output is quantised online, reusing work the kernel already does, and the
quantisation runs per wavefront on 32 x 32 blocks.

The number format is the public OCP Microscaling Formats (MX) Specification
v1.0 (Open Compute Project), sections on the MXFP8 E4M3 element type, the
E8M0 scale type and the conversion of a vector of fp32 values to an MX block:
  * E4M3 element: sign, 4 exponent bits with bias 7, 3 mantissa bits,
    subnormals, no infinities; S.1111.111 is NaN; the largest finite
    magnitude is 448 = 1.75 * 2^8.
  * E8M0 scale: an 8-bit biased exponent e, value 2^(e - 127), e in 0..254.
  * One scale per block of 32 values: X = 2^(floor(log2(max |v|)) - 8), 8
    being the largest E4M3 exponent; each element is v / X rounded to the
    nearest E4M3 value, ties to even mantissa, magnitudes beyond 448 clamped
    to 448.

Readings of what the pages leave open (each repeated where it is used):
  R1 operands: Q and K are quantised in blocks of 32 consecutive head-dim
     elements (the contraction of Q K^T); V in blocks of 32 consecutive keys
     of a sequence, counted from its first key, per head and head-dim column
     (the contraction of P V); P in blocks of 32 consecutive keys of a row,
     counted from the sequence's first key.  head_dim must be a multiple of
     32.
  R2 online quantisation of P: the weight of a visible key is 2^(t - m) with
     t = scale * log2(e) * q.k and m the row max rounded up to an integer (the
     max the kernel keeps anyway).  With m an integer, the block scale is
     2^(floor(tb) - m - 8) and the elements are 2^(t - floor(tb) + 8), tb being
     the block's largest visible t: the codes depend on the scores alone, and
     m enters only the scale.  Invisible keys weigh 0 and take no part in tb;
     a block without visible keys is all zero.
  R3 the softmax denominator and the lse use the exact weights 2^(t - m);
     only the P operand of P V is quantised.
  R4 a block whose floor(log2 max) - 8 is below -127 takes the scale 2^-127
     (the smallest E8M0 value); an all-zero block has scale 2^-127 and zero
     elements.
  R5 out and lse as in attention.attention_fwd (rows without a visible key:
     out = 0, lse = -inf; causal cross attention bottom-right aligned).
  R6 backward (mx_attention_bwd): each product's operands in MX blocks along
     its contraction axis -- S = Q K^T and dP = dO V^T over the head
     dimension (row images), dV = P^T dO and dK = dS^T Q over queries
     (blocks of 32 queries counted from the sequence's first one: P and dS
     per key column, dO and Q per column), dQ = dS K over keys (dS per query
     row, K per column).
  R7 P is recomputed from the forward's lse in full precision (as the
     plain backward does), delta = rowsum(dO o O) from the given O and dO,
     and dS = P o (dP - delta) is formed before either of its
     quantisations.
  R8 P and dS take the smallest power-of-two scale that keeps their block
     unsaturated: 2^k with k the least integer for which max|x| <= 448 2^k
     (e8m0_exponent_fit), not the vector conversion's 2^(floor(log2 max) -
     8).  The latter saturates block maxima in (1.75, 2) x 2^j, and its
     threshold sits exactly at P = 1, the weight of every row with a single
     visible key (the first query of causal self attention): the last bit
     of P's evaluation would decide between 1 and 0.875.  The fitted scale's
     threshold is max = 448 2^k (P = 0.875 2^j), where weights do not
     gather, and nothing saturates.
"""

import math

import numpy as np

from .attention import visible_mask

E4M3_MAX = 448.0
E4M3_EMAX = 8        # exponent of the largest E4M3 binade
E8M0_BIAS = 127
E8M0_MIN_EXP = -127
E8M0_MAX_EXP = 127
BLOCK = 32


def e4m3_decode(codes):
    """Value of each E4M3 code (OCP MX v1.0, E4M3 element type): NaN for
    0x7F / 0xFF, subnormals 2^-6 * m/8 for exponent field 0."""
    c = np.asarray(codes, dtype=np.int64)
    sign = np.where(c & 0x80, -1.0, 1.0)
    e = (c >> 3) & 0xF
    m = (c & 7).astype(np.float64)
    mag = np.where(e == 0, m / 8.0 * 2.0 ** -6, (1.0 + m / 8.0) * np.exp2(e - 7.0))
    mag = np.where((e == 15) & (c & 7 == 7), np.nan, mag)
    return sign * mag


def _round_half_even(x):
    """Nearest integer, ties to even, for non-negative fp64 x."""
    f = np.floor(x)
    r = x - f
    up = (r > 0.5) | ((r == 0.5) & (np.mod(f, 2) == 1))
    return f + up


def e4m3_encode(x):
    """Nearest E4M3 code of each finite value (ties to even mantissa),
    magnitudes beyond 448 clamped to 448 (OCP MX v1.0, conversion to the
    element type).  The sign of zero is kept."""
    x = np.asarray(x, dtype=np.float64)
    if not np.all(np.isfinite(x)):
        raise ValueError("e4m3_encode takes finite values")
    sign = np.where(np.signbit(x), 0x80, 0).astype(np.int64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    code = np.zeros(a.shape, dtype=np.int64)
    normal = a >= 2.0 ** -6
    # subnormal range: multiples of 2^-9; rounding up to 8 * 2^-9 = 2^-6 gives
    # code 8, which is also the smallest normal's code
    sub = ~normal
    code[sub] = _round_half_even(a[sub] * 2.0 ** 9).astype(np.int64)
    if np.any(normal):
        an = a[normal]
        e = np.floor(np.log2(an)).astype(np.int64)
        # log2 of a value just below a power of two may round up to it
        e = np.where(np.exp2(e.astype(np.float64)) > an, e - 1, e)
        n = _round_half_even(an / np.exp2(e - 3.0)).astype(np.int64)   # in 8 .. 16
        carry = n == 16
        e = np.where(carry, e + 1, e)
        n = np.where(carry, 8, n)
        code[normal] = ((e + 7) << 3) | (n - 8)
    return (sign | code).astype(np.uint8)


def e8m0_exponent(amax):
    """Shared exponent of a block with largest magnitude amax (OCP MX v1.0,
    vector conversion): floor(log2 amax) - 8, clamped to the E8M0 range
    (R4); an all-zero block takes the smallest exponent."""
    amax = np.asarray(amax, dtype=np.float64)
    out = np.full(amax.shape, E8M0_MIN_EXP, dtype=np.int64)
    pos = amax > 0
    if np.any(pos):
        a = amax[pos]
        e = np.floor(np.log2(a)).astype(np.int64)
        e = np.where(np.exp2(e.astype(np.float64)) > a, e - 1, e)
        out[pos] = np.clip(e - E4M3_EMAX, E8M0_MIN_EXP, E8M0_MAX_EXP)
    return out


def mx_quantize_block(v):
    """One MX block: (codes uint8 [n], exponent int) of a 1-D array of at
    most 32 values (OCP MX v1.0, conversion of a vector to an MX block)."""
    v = np.asarray(v, dtype=np.float64)
    if v.ndim != 1 or v.size > BLOCK:
        raise ValueError("a block is a 1-D array of at most 32 values")
    ex = int(e8m0_exponent(np.max(np.abs(v), initial=0.0)))
    return e4m3_encode(v / 2.0 ** ex), ex


def mx_quantize_rows(x):
    """R1, Q and K: blocks of 32 consecutive elements of the last axis.

    x [T, H, d] -> (codes uint8 [T, H, d], exps int64 [T, H, d // 32])."""
    x = np.asarray(x, dtype=np.float64)
    T, H, d = x.shape
    if d % BLOCK:
        raise ValueError("head_dim must be a multiple of 32")
    blocks = x.reshape(T, H, d // BLOCK, BLOCK)
    exps = e8m0_exponent(np.max(np.abs(blocks), axis=3))
    codes = e4m3_encode(blocks / np.exp2(exps[..., None].astype(np.float64)))
    return codes.reshape(T, H, d), exps


def mx_quantize_keys(x, offsets):
    """R1, V: blocks of 32 consecutive rows of a sequence, counted from its
    first row, per head and column (the last block of a sequence may be
    shorter).

    x [T, H, d] -> (codes uint8 [T, H, d], exps int64 [T, H, d]): exps[r] is
    the exponent of the block holding row r."""
    x = np.asarray(x, dtype=np.float64)
    off = np.asarray(offsets, dtype=np.int64)
    codes = np.zeros(x.shape, dtype=np.uint8)
    exps = np.zeros(x.shape, dtype=np.int64)
    for b in range(len(off) - 1):
        for r0 in range(int(off[b]), int(off[b + 1]), BLOCK):
            r1 = min(r0 + BLOCK, int(off[b + 1]))
            blk = x[r0:r1]                                   # [n, H, d]
            ex = e8m0_exponent(np.max(np.abs(blk), axis=0))  # [H, d]
            codes[r0:r1] = e4m3_encode(blk / np.exp2(ex.astype(np.float64))[None])
            exps[r0:r1] = ex[None]
    return codes, exps


def mx_dequantize_rows(codes, exps):
    """Values of mx_quantize_rows' output."""
    T, H, d = codes.shape
    v = e4m3_decode(codes).reshape(T, H, d // BLOCK, BLOCK)
    return (v * np.exp2(np.asarray(exps, dtype=np.float64))[..., None]).reshape(T, H, d)


def mx_dequantize_keys(codes, exps):
    """Values of mx_quantize_keys' output."""
    return e4m3_decode(codes) * np.exp2(np.asarray(exps, dtype=np.float64))


def quantize_p(t, vis):
    """R2: the quantised softmax numerator of one (sequence, head) block.

    t [lq, lk]: scale * log2(e) * q.k;  vis: visibility.  Returns
    (codes uint8 [lq, lk], fb int64 [lq, nblocks]) where key j of row i
    weighs e4m3_decode(codes[i, j]) * 2^(fb[i, j // 32] - 8) relative to the
    row max (the factor 2^-m of R2 is left to the caller).  Blocks without a
    visible key have codes 0 and fb 0."""
    lq, lk = t.shape
    nb = (lk + BLOCK - 1) // BLOCK
    codes = np.zeros((lq, lk), dtype=np.uint8)
    fb = np.zeros((lq, nb), dtype=np.int64)
    for c in range(nb):
        j0, j1 = BLOCK * c, min(BLOCK * c + BLOCK, lk)
        tb = t[:, j0:j1]
        vb = vis[:, j0:j1]
        live = vb.any(axis=1)
        bmax = np.where(vb, tb, -np.inf).max(axis=1)
        f = np.where(live, np.floor(np.where(live, bmax, 0.0)), 0.0)
        el = np.exp2(np.where(vb, tb - f[:, None] + E4M3_EMAX, -np.inf))
        codes[:, j0:j1] = np.where(vb, e4m3_encode(el), 0)
        fb[:, c] = f.astype(np.int64)
    return codes, fb


def mx_attention_fwd(q, k, v, q_offsets, kv_offsets, scale, causal=False):
    """MXFP8 jagged softmax attention forward (R1 - R5), fp64 arithmetic on
    the quantised operands.

    q [T_q, H, d], k / v [T_k, H, d] (the bf16 inputs, as floats);
    returns (out [T_q, H, d], lse [H, T_q])."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    if qo[-1] != q.shape[0] or ko[-1] != k.shape[0] or v.shape != k.shape or q.shape[1:] != k.shape[1:]:
        raise ValueError("offsets do not match the value tensors")
    qh = mx_dequantize_rows(*mx_quantize_rows(q))
    kh = mx_dequantize_rows(*mx_quantize_rows(k))
    vh = mx_dequantize_keys(*mx_quantize_keys(v, ko))
    T_q, H, d = q.shape
    out = np.zeros((T_q, H, d))
    lse = np.full((H, T_q), -np.inf)
    c = scale / math.log(2.0)   # scale * log2(e)
    for b in range(len(qo) - 1):
        qs, qe, ks, ke = int(qo[b]), int(qo[b + 1]), int(ko[b]), int(ko[b + 1])
        lq, lk = qe - qs, ke - ks
        if lq == 0 or lk == 0:
            continue
        vis = visible_mask(lq, lk, causal)
        live = vis.any(axis=1)
        for h in range(H):
            t = c * (qh[qs:qe, h] @ kh[ks:ke, h].T)
            m = np.where(live, np.where(vis, t, -np.inf).max(axis=1), 0.0)
            w = np.where(vis, np.exp2(t - m[:, None]), 0.0)          # R3: exact weights
            den = w.sum(axis=1)
            codes, fb = quantize_p(t, vis)
            blk = np.arange(lk) // BLOCK
            pq = e4m3_decode(codes) * np.exp2(fb[:, blk] - E4M3_EMAX - m[:, None])
            o = pq @ vh[ks:ke, h]
            out[qs:qe, h] = np.where(live[:, None], o / np.where(live, den, 1.0)[:, None], 0.0)
            with np.errstate(divide="ignore"):
                lse[h, qs:qe] = np.where(live, (m + np.log2(np.where(live, den, 1.0))) * math.log(2.0), -np.inf)
    return out, lse


# ------------------------------------------------------------------ backward

def e8m0_exponent_fit(amax):
    """Block exponent of P and dS (R8): the least integer k with amax <= 448
    2^k, clamped to the E8M0 range; an all-zero block takes the smallest
    exponent.  The block's largest element then lies in [224, 448]."""
    amax = np.asarray(amax, dtype=np.float64)
    k = e8m0_exponent(amax)   # floor(log2 amax) - 8: amax in [256, 512) x 2^k
    k = np.where((amax > 0) & (amax > E4M3_MAX * np.exp2(k.astype(np.float64))), k + 1, k)
    return np.clip(k, E8M0_MIN_EXP, E8M0_MAX_EXP)


def mx_quantize_matrix(x, axis):
    """MX blocks of 32 consecutive entries of a 2-D block along `axis` (0:
    down each column, 1: along each row), counted from index 0, with the
    fitted block exponent (R8); returns the dequantised values (the weights
    and dS of one (sequence, head) along queries or along keys)."""
    x = np.asarray(x, dtype=np.float64)
    y = x if axis == 0 else x.T
    out = np.zeros_like(y)
    for r0 in range(0, y.shape[0], BLOCK):
        blk = y[r0:r0 + BLOCK]
        ex = e8m0_exponent_fit(np.max(np.abs(blk), axis=0))
        sc = np.exp2(ex.astype(np.float64))[None]
        out[r0:r0 + BLOCK] = e4m3_decode(e4m3_encode(blk / sc)) * sc
    return out if axis == 0 else out.T


def mx_attention_bwd(q, k, v, out, dout, lse, q_offsets, kv_offsets, scale, causal=False, quantize=True):
    """MXFP8 jagged softmax attention backward (R6 - R8), fp64 arithmetic on
    the quantised operands.

    out, lse: the forward's outputs (as jfa_backward takes them).  Each
    product's operands are quantised along its contraction axis:
      dP = dO V^T, S = Q K^T   over the head dimension: row images;
      dV = P^T dO, dK = dS^T Q over queries: P and dS per key column, dO and
                               Q per column, blocks of 32 queries;
      dQ = dS K                over keys: dS per query row, K per column,
                               blocks of 32 keys.
    P = exp(scale S - lse) from the quantised S, in full precision, and
    dS = P o (dP - delta), delta = rowsum(dO o O), before their own
    quantisation.  quantize=False replaces every quantisation by the
    identity (the plain attention backward; a structural pin)."""
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    out = np.asarray(out, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    lse = np.asarray(lse, dtype=np.float64)
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    if quantize:
        rows = lambda x: mx_dequantize_rows(*mx_quantize_rows(x))          # noqa: E731
        seq = lambda x, o: mx_dequantize_keys(*mx_quantize_keys(x, o))     # noqa: E731
        mat = mx_quantize_matrix
    else:
        rows = lambda x: x                                                  # noqa: E731
        seq = lambda x, o: x                                                # noqa: E731
        mat = lambda x, axis: x                                             # noqa: E731
    q_r, k_r, v_r, do_r = rows(q), rows(k), rows(v), rows(dout)
    q_c, do_c, k_c = seq(q, qo), seq(dout, qo), seq(k, ko)
    delta = (dout * out).sum(axis=2)   # [T_q, H]
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    H = q.shape[1]
    for b in range(len(qo) - 1):
        qs, qe, ks, ke = int(qo[b]), int(qo[b + 1]), int(ko[b]), int(ko[b + 1])
        lq, lk = qe - qs, ke - ks
        if lq == 0 or lk == 0:
            continue
        vis = visible_mask(lq, lk, causal)
        for h in range(H):
            s = scale * (q_r[qs:qe, h] @ k_r[ks:ke, h].T)
            lrow = lse[h, qs:qe]
            p = np.where(vis & np.isfinite(lrow)[:, None], np.exp(s - np.where(np.isfinite(lrow), lrow, 0.0)[:, None]),
                         0.0)
            dv[ks:ke, h] = mat(p, 0).T @ do_c[qs:qe, h]
            dp = do_r[qs:qe, h] @ v_r[ks:ke, h].T
            ds = p * (dp - delta[qs:qe, h][:, None])
            dk[ks:ke, h] = scale * (mat(ds, 0).T @ q_c[qs:qe, h])
            dq[qs:qe, h] = scale * (mat(ds, 1) @ k_c[ks:ke, h])
    return dq, dk, dv
