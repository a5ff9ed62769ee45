"""Plain fp64 jagged attention: the definition, one sequence and head at a time.

TEST INFRASTRUCTURE ONLY (see the package docstring for the rule and for the
citation keys used below).

Layout of the jagged tensors (values packed by sequence, no padding):
  q, out, dq      : [T_q, H, d]   rows qo[b] .. qo[b+1]-1 belong to sequence b
  k, v, dk, dv    : [T_k, H, d]   rows ko[b] .. ko[b+1]-1 belong to sequence b
  lse             : [H, T_q]      natural-log log-sum-exp of the scaled scores
Offsets are monotone integer arrays of length B+1 starting at 0.

Readings of points the pages leave open (each is stated where it is used):
  * causal with Lq != Lk is bottom-right aligned: query i of a sequence sees
    key j iff j <= i + (Lk - Lq); this is j <= i for self attention.
  * a softmax row with no visible key has out = 0 and lse = -inf.
  * the GDPA activation is silu(s * q.k) / Lk, Lk being the sequence's own key
    count (also under causal masking); invisible entries weigh 0.
  * BlockAttention's fixed blocks ([GEM-MFU, Detailed notes: BlockAttention])
    are read as: self attention in which every run of `block` consecutive
    tokens of a sequence, counted from its first token, attends only within
    itself -- each block is a sequence of its own (so the GDPA normaliser is
    the block's key count, and causal masking applies inside the block).
"""

import numpy as np

ACTIVATIONS = ("softmax", "silu")


def visible_mask(lq, lk, causal):
    """Boolean [lq, lk] visibility of key j to query i.

    [GEM-MFU, Detailed notes: jagged input] lists self and asymmetric-QKV cross
    attention; causal masking of a cross pair is read bottom-right aligned.
    """
    i = np.arange(lq)[:, None]
    j = np.arange(lk)[None, :]
    if causal:
        return j <= i + (lk - lq)
    return np.ones((lq, lk), dtype=bool)


def _sigmoid(x):
    # Two-branch form so that neither branch overflows.
    out = np.empty_like(x)
    pos = x >= 0
    out[pos] = 1.0 / (1.0 + np.exp(-x[pos]))
    e = np.exp(x[~pos])
    out[~pos] = e / (1.0 + e)
    return out


def _segments(qo, ko, block):
    """(q start, q end, k start, k end) of every attention unit: the sequences,
    or with block > 0 the consecutive `block`-token runs of each sequence
    ([GEM-MFU, Detailed notes: BlockAttention]: fixed blocks of 64 tokens,
    which turn the cost from quadratic to linear in the length)."""
    segs = []
    for b in range(len(qo) - 1):
        qs, qe, ks, ke = qo[b], qo[b + 1], ko[b], ko[b + 1]
        if block <= 0:
            segs.append((qs, qe, ks, ke))
            continue
        if qe - qs != ke - ks:
            raise ValueError("block attention is self attention: equal query and key lengths")
        for c in range(0, qe - qs, block):
            n = min(block, qe - qs - c)
            segs.append((qs + c, qs + c + n, ks + c, ks + c + n))
    return segs


def _check(q, k, v, q_offsets, kv_offsets, activation):
    if activation not in ACTIVATIONS:
        raise ValueError("activation must be one of %r" % (ACTIVATIONS,))
    qo = np.asarray(q_offsets, dtype=np.int64)
    ko = np.asarray(kv_offsets, dtype=np.int64)
    if qo.ndim != 1 or ko.shape != qo.shape or qo[0] != 0 or ko[0] != 0:
        raise ValueError("offsets must be 1-D, equal length, starting at 0")
    if np.any(np.diff(qo) < 0) or np.any(np.diff(ko) < 0):
        raise ValueError("offsets must be non-decreasing")
    if qo[-1] != q.shape[0] or ko[-1] != k.shape[0] or v.shape != k.shape:
        raise ValueError("offsets do not match the value tensors")
    if q.shape[1:] != k.shape[1:]:
        raise ValueError("q and k must share heads and head_dim")
    return qo, ko


def _probs(S, vis, activation, lk):
    """Attention weights of one (sequence, head) block, plus lse for softmax.

    softmax: [GEM-MFU, Detailed notes: JFA] -- exact softmax over the visible
    keys of each row; masked keys weigh exactly 0.
    silu:    [GEM-MFU, Detailed notes: GDPA] -- non-softmax activation,
    silu(S)/Lk on visible entries, 0 elsewhere.
    """
    if activation == "softmax":
        live = vis.any(axis=1)
        m = np.where(vis, S, -np.inf).max(axis=1, initial=-np.inf)
        m = np.where(live, m, 0.0)
        e = np.exp(np.where(vis, S - m[:, None], -np.inf))
        total = e.sum(axis=1)
        P = e / np.where(live, total, 1.0)[:, None]
        with np.errstate(divide="ignore"):
            lse = np.where(live, m + np.log(np.where(live, total, 1.0)), -np.inf)
        return P, lse
    A = np.where(vis, S * _sigmoid(S) / max(lk, 1), 0.0)
    return A, None


def _rope_inputs(q, k, qo, ko, rope_base):
    """Q and K rotated at their positions within their sequences (see
    oracle.rope; [GEM-MFU, Detailed notes: BlockAttention item])."""
    from .rope import rope, sequence_positions
    return rope(q, sequence_positions(qo), rope_base), rope(k, sequence_positions(ko), rope_base)


def attention_fwd(q, k, v, q_offsets, kv_offsets, scale, activation="softmax", causal=False, block=0,
                  rope_base=None):
    """Jagged attention forward in fp64.

    Returns (out [T_q, H, d], lse [H, T_q] or None for silu).
    [GEM-MFU, Detailed notes: JFA] for softmax, [GEM-MFU, Detailed notes: GDPA]
    for silu; every sequence is independent of the others
    ([GEM-MFU, Detailed notes: jagged input]).  block > 0: BlockAttention,
    attention within each `block`-token run of a sequence (see _segments).
    rope_base: Q and K first rotated by the rotary embedding of that base
    at their positions within their sequences (oracle.rope).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    qo, ko = _check(q, k, v, q_offsets, kv_offsets, activation)
    if rope_base is not None:
        q, k = _rope_inputs(q, k, qo, ko, rope_base)
    T_q, H, d = q.shape
    out = np.zeros((T_q, H, v.shape[2]))
    lse = np.full((H, T_q), -np.inf) if activation == "softmax" else None
    for qs, qe, ks, ke in _segments(qo, ko, block):
        lq, lk = qe - qs, ke - ks
        if lq == 0:
            continue
        vis = visible_mask(lq, lk, causal)
        for h in range(H):
            Q, K, V = q[qs:qe, h], k[ks:ke, h], v[ks:ke, h]
            S = scale * (Q @ K.T)
            P, row_lse = _probs(S, vis, activation, lk)
            out[qs:qe, h] = P @ V
            if lse is not None:
                lse[h, qs:qe] = row_lse
    return out, lse


def attention_bwd(q, k, v, dout, q_offsets, kv_offsets, scale, activation="softmax", causal=False, block=0,
                  rope_base=None):
    """Gradients (dq, dk, dv) of sum(out * dout) for the forward above, fp64.

    The chain rule written out per (sequence, head) block:
      softmax: dV = P^T dO, dP = dO V^T, dS = P o (dP - rowsum(P o dP)),
      silu:    dV = A^T dO, dA = dO V^T, dS = dA o silu'(S) / Lk on visible
               entries, silu'(x) = sig(x) (1 + x (1 - sig(x))),
      both:    dQ = scale dS K, dK = scale dS^T Q.
    The backward's parallel split without atomics ([GEM-MFU, Detailed notes:
    JFA]) changes only how these sums are formed, not their values.  block:
    as in attention_fwd.  rope_base: the gradients are those of the rotated
    Q and K turned back, dq = R(p)^T dq' (oracle.rope, inverse).
    """
    q = np.asarray(q, dtype=np.float64)
    k = np.asarray(k, dtype=np.float64)
    v = np.asarray(v, dtype=np.float64)
    dout = np.asarray(dout, dtype=np.float64)
    qo, ko = _check(q, k, v, q_offsets, kv_offsets, activation)
    if rope_base is not None:
        from .rope import rope, sequence_positions
        qr, kr = _rope_inputs(q, k, qo, ko, rope_base)
        dq, dk, dv = attention_bwd(qr, kr, v, dout, qo, ko, scale, activation, causal, block)
        return (rope(dq, sequence_positions(qo), rope_base, inverse=True),
                rope(dk, sequence_positions(ko), rope_base, inverse=True), dv)
    if dout.shape != q.shape[:2] + (v.shape[2],):
        raise ValueError("dout must have the shape of out")
    T_q, H, d = q.shape
    dq = np.zeros_like(q)
    dk = np.zeros_like(k)
    dv = np.zeros_like(v)
    for qs, qe, ks, ke in _segments(qo, ko, block):
        lq, lk = qe - qs, ke - ks
        if lq == 0 or lk == 0:
            continue
        vis = visible_mask(lq, lk, causal)
        for h in range(H):
            Q, K, V, dO = q[qs:qe, h], k[ks:ke, h], v[ks:ke, h], dout[qs:qe, h]
            S = scale * (Q @ K.T)
            P, _ = _probs(S, vis, activation, lk)
            dv[ks:ke, h] = P.T @ dO
            dP = dO @ V.T
            if activation == "softmax":
                dS = P * (dP - (P * dP).sum(axis=1, keepdims=True))
            else:
                sig = _sigmoid(S)
                dS = np.where(vis, dP * sig * (1.0 + S * (1.0 - sig)) / lk, 0.0)
            dq[qs:qe, h] = scale * (dS @ K)
            dk[ks:ke, h] = scale * (dS.T @ Q)
    return dq, dk, dv
