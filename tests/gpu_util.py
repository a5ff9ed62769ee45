"""Helpers of the GPU tests: move a drawn batch to the device, run the HIP
path through the C ABI binding, and compare with the CPU oracle."""

import math

import numpy as np
import torch

import oracle
from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import bf16_bits_to_f64, offsets_from_lengths

FWD_ATOL = 1e-2      # forward max abs error of the arithmetic vs the fp64 oracle
FWD_ATOL_FP32 = 1e-4   # the same for fp32 inputs (fp32 operands and weights throughout)
LSE_ATOL = 1e-3      # lse abs error (fp32 kernel value vs fp64)
GRAD_RTOL = 2e-2     # relative L2 error of dq, dk, dv: per tensor and per sequence
GRAD_RTOL_FP32 = 1e-4  # the same for fp32 inputs
# Per-sequence gate: a sequence's reference norm is floored at this fraction
# of what an average sequence of its size has (its share of the tensor's
# norm), so that sequences whose gradient cancels (one key gives dq = 0
# exactly) are measured against the tensor's scale instead of their own
# tiny norm.  At 1e-2 the fp32 path's rounding in such a sequence (about
# 1e-6 of its share) read as 1.2e-4 against the 1e-4 gate; at 1e-1 a
# one-key sequence of a pooled fp32 batch (1166 keys, dk exactly 0, a
# residue of 2.5e-6 = 4e-7 of the cancelling terms scale * dP * q) read as
# 1.06e-4: the residue scales with the cancelling terms, which can be ten
# times an average row's gradient.
SEQ_NORM_FLOOR = 3e-1
# ... and at this fraction of the norm of its own term magnitudes (sums of
# |terms| of each gradient element, grad_term_magnitudes).  A gradient of n
# terms of random sign has about 1/sqrt(n) of their magnitude (0.34 at 260
# terms, 0.056 at 2000, measured), so below some 10^4 terms the floor is
# under the sequence's own norm and changes nothing.  Where the terms
# cancel -- dK and dQ with one key, where the fp32 path's residue read as
# 7e-4 against the share floor (one key, 31 queries) -- the residue is
# 3e-9 to 7e-7 of the
# magnitudes (a plain float32 backward), so at most 7e-5 against this
# floor, while an error that breaks the cancellation reads as its
# fraction of the magnitudes times 100.
MAG_FLOOR = 1e-2


def dev():
    return torch.device("cuda:0")


def values_to_device(arr, dtype):
    if dtype == "bf16":
        return torch.from_numpy(np.ascontiguousarray(arr).view(np.int16)).view(torch.bfloat16).to(dev())
    return torch.from_numpy(np.ascontiguousarray(arr, dtype=np.float32)).to(dev())


def to_f64(t):
    if t.dtype == torch.bfloat16:
        return bf16_bits_to_f64(t.view(torch.int16).cpu().numpy().view(np.uint16))
    return t.double().cpu().numpy()


class Dev:
    """A batch on the device."""

    def __init__(self, batch):
        self.b = batch
        wl = batch.workload
        self.dtype = wl.dtype
        self.q = values_to_device(batch.q, wl.dtype)
        self.k = values_to_device(batch.k, wl.dtype)
        self.v = values_to_device(batch.v, wl.dtype)
        self.do = values_to_device(batch.dout, wl.dtype) if batch.dout is not None else None
        self.qo = torch.from_numpy(batch.q_offsets.astype(np.int32)).to(dev())
        self.ko = torch.from_numpy(batch.kv_offsets.astype(np.int32)).to(dev())
        self.mq = int(batch.q_lengths.max()) if len(batch.q_lengths) else 0
        self.mk = int(batch.kv_lengths.max()) if len(batch.kv_lengths) else 0
        self.scale = 1.0 / math.sqrt(wl.head_dim)
        self.act = wl.activation
        self.causal = wl.causal

    def forward(self):
        return jfa.forward(self.q, self.k, self.v, self.qo, self.ko, self.mq, self.mk, self.scale, self.act,
                           self.causal)

    def backward(self, out, lse):
        return jfa.backward(self.q, self.k, self.v, out, self.do, lse, self.qo, self.ko, self.mq, self.mk,
                            self.scale, self.act, self.causal)


def oracle_fwd(batch, seqs=None):
    """Oracle forward, for all sequences or only those in `seqs` (returns
    arrays restricted to those sequences' rows, plus the row index maps)."""
    wl = batch.workload
    s = 1.0 / math.sqrt(wl.head_dim)
    q, k, v = batch.f64("q"), batch.f64("k"), batch.f64("v")
    qo, ko = batch.q_offsets, batch.kv_offsets
    if seqs is None:
        return oracle.attention_fwd(q, k, v, qo, ko, s, wl.activation, wl.causal)
    qi, ki, qs, ks = _subset(batch, seqs)
    return oracle.attention_fwd(q[qi], k[ki], v[ki], qs, ks, s, wl.activation, wl.causal)


def oracle_bwd(batch, seqs=None):
    wl = batch.workload
    s = 1.0 / math.sqrt(wl.head_dim)
    q, k, v, do = batch.f64("q"), batch.f64("k"), batch.f64("v"), batch.f64("dout")
    qo, ko = batch.q_offsets, batch.kv_offsets
    if seqs is None:
        return oracle.attention_bwd(q, k, v, do, qo, ko, s, wl.activation, wl.causal)
    qi, ki, qs, ks = _subset(batch, seqs)
    return oracle.attention_bwd(q[qi], k[ki], v[ki], do[qi], qs, ks, s, wl.activation, wl.causal)


def _subset(batch, seqs):
    qo, ko = batch.q_offsets, batch.kv_offsets
    qi = np.concatenate([np.arange(qo[b], qo[b + 1]) for b in seqs]).astype(np.int64)
    ki = np.concatenate([np.arange(ko[b], ko[b + 1]) for b in seqs]).astype(np.int64)
    qs = offsets_from_lengths([qo[b + 1] - qo[b] for b in seqs])
    ks = offsets_from_lengths([ko[b + 1] - ko[b] for b in seqs])
    return qi, ki, qs, ks


def rows_of(batch, seqs, side="q"):
    o = batch.q_offsets if side == "q" else batch.kv_offsets
    return np.concatenate([np.arange(o[b], o[b + 1]) for b in seqs]).astype(np.int64)


def half_ulp_bf16(x):
    """Half a bf16 unit in the last place at |x| (8 significant bits)."""
    ax = np.maximum(np.abs(x), np.finfo(np.float32).tiny)
    return np.exp2(np.floor(np.log2(ax)) - 8.0)


def forward_tolerance(ref_out, dtype, extra=None):
    """Per-element bound on |out - ref|.  fp32: 1e-4 flat.  bf16: 1e-2 flat
    for |ref| < 2; above that the stored bf16 output alone is off by up to
    half a bf16 ulp of the value (0.0078 at 2, 0.0156 at 4: more than a flat
    1e-2 leaves for the arithmetic), so there the bound is 1e-2 plus half an
    ulp.  extra: a per-element arithmetic bound added to the flat one
    (which then holds below |ref| + extra = 2).  The ulp is taken where the
    unrounded kernel value can reach, |ref| + 1e-2 + extra, in case the
    rounding crosses into the next binade."""
    e = 0.0 if extra is None else extra
    if dtype == torch.bfloat16:
        a = np.abs(ref_out)
        return FWD_ATOL + e + np.where(a + e < 2.0, 0.0, half_ulp_bf16(a + FWD_ATOL + e))
    return FWD_ATOL_FP32 + e


def silu_weight_rounding(q, k, v, q_offsets, kv_offsets, scale, causal):
    """Per-element bound [T_q, H, d] on what rounding the SiLU weights to
    bf16 for the P V product moves the output by (q, k, v float64 [T, H, d],
    the rows the kernel multiplies; sequence b owns rows q_offsets[b] ..
    and kv_offsets[b] ..): each weight w_ij = silu(scale q_i.k_j) / L_kv is
    rounded to 8 significant bits, which moves it by up to half a unit in
    its last place: 2^-8 of it just above a power of two (4.0767 -> 4.0625),
    so out_ic moves by at most 2^-8 sum_j |w_ij| |v_jc|.  The softmax
    weights are normalised (a convex combination of V rows, the flat 1e-2
    covers them); SiLU's are not, and with few keys |out| reaches several
    units, where 2^-8 of it exceeds the flat 1e-2."""
    out = np.zeros(q.shape)
    for b in range(len(q_offsets) - 1):
        q0, q1, k0, k1 = int(q_offsets[b]), int(q_offsets[b + 1]), int(kv_offsets[b]), int(kv_offsets[b + 1])
        if q1 == q0 or k1 == k0:
            continue
        s = np.einsum("ihc,jhc->hij", q[q0:q1], k[k0:k1]) * scale
        w = np.abs(s / (1.0 + np.exp(-s))) / (k1 - k0)
        if causal:
            i = np.arange(q1 - q0)[:, None]
            j = np.arange(k1 - k0)[None, :]
            w = np.where((j <= i + (k1 - k0) - (q1 - q0))[None], w, 0.0)
        out[q0:q1] = np.einsum("hij,jhc->ihc", w, np.abs(v[k0:k1]))
    return 2.0 ** -8 * out


def silu_weight_rounding_of(batch):
    """silu_weight_rounding for a jagged batch as the jagged calls take it."""
    return silu_weight_rounding(batch.f64("q"), batch.f64("k"), batch.f64("v"), batch.q_offsets,
                                batch.kv_offsets, batch.scale, batch.workload.causal)


def rope_lse_bound(q, k, offsets, block, causal, scale):
    """Per (head, row) bound on |lse_gpu - lse_ref| when Q and K are turned by
    the rotary embedding and the turned values rounded to bf16 before the
    products: each rounding moves a value by at most 2^-8 of itself (half a
    unit in the last of 8 significant bits, just above a power of two), so a
    score moves by at most scale * 2^-7 * sum_c |q'_c| |k'_c|, and a turned
    pair (c, c + d/2) keeps its length, which bounds that sum by the pair
    lengths of the unturned rows (Cauchy-Schwarz).  lse is a smooth maximum
    of the row's scores: its error is at most the largest score error.
    Returns LSE_ATOL plus that bound for every visible row (q, k fp64
    [T, H, d]; self attention within `block`-token runs)."""
    T, H, d = q.shape
    h = d // 2
    qn = np.sqrt(q[..., :h] ** 2 + q[..., h:] ** 2)   # [T, H, d/2] pair lengths
    kn = np.sqrt(k[..., :h] ** 2 + k[..., h:] ** 2)
    out = np.full((H, T), LSE_ATOL)
    off = np.asarray(offsets, dtype=np.int64)
    for b in range(len(off) - 1):
        for c0 in range(off[b], off[b + 1], block):
            c1 = min(c0 + block, off[b + 1])
            m = np.einsum("ihc,jhc->hij", qn[c0:c1], kn[c0:c1])   # [H, rows, keys]
            if causal:
                m = np.where(np.tril(np.ones((c1 - c0, c1 - c0), dtype=bool))[None], m, 0.0)
            out[:, c0:c1] += scale * 2.0 ** -7 * m.max(axis=2)
    return out


def rope_rounding_effect(q, k, v, offsets, block, scale, activation, causal, base):
    """Per-element [T, H, d] effect on the output of the BlockAttention
    kernels' rounding of the turned Q and K to bf16 before the products:
    |attention(bf16(q'), bf16(k'), v) - attention(q', k', v)|, both by the
    oracle's block attention in fp64, with q' and k' turned at their
    positions within their `block`-token runs as the kernels turn them (any
    origin gives the same attention in exact arithmetic, not the same
    roundings).  q, k, v float64 [T, H, d]; self attention, sequence b owns
    rows offsets[b] .."""
    import oracle
    from oracle.rope import rope as turn
    off = np.asarray(offsets, dtype=np.int64)
    pos = np.concatenate([np.arange(int(off[i + 1] - off[i])) % block for i in range(len(off) - 1)] +
                         [np.zeros(0, np.int64)])
    as_bf16 = lambda x: torch.from_numpy(np.ascontiguousarray(x)).to(torch.bfloat16).double().numpy()  # noqa: E731
    qr, kr = as_bf16(turn(q, pos, base)), as_bf16(turn(k, pos, base))
    emu, _ = oracle.attention_fwd(qr, kr, v, off, off, scale, activation, causal, block=block)
    exact, _ = oracle.attention_fwd(q, k, v, off, off, scale, activation, causal, block=block, rope_base=base)
    return np.abs(emu - exact)


def check_forward(out, lse, ref_out, ref_lse, activation, q_rows=None, lse_atol=None, extra_tol=None):
    """Gates the forward; returns the flat max abs error over all elements
    (printed: the per-magnitude bound above is what is gated).  lse_atol:
    a per-element lse bound [H, rows] instead of LSE_ATOL; extra_tol: a
    per-element bound added to the output's (silu_weight_rounding)."""
    o = to_f64(out)
    if q_rows is not None:
        o = o[q_rows]
    diff = np.abs(o - ref_out)
    err = float(diff.max()) if o.size else 0.0
    tol = forward_tolerance(ref_out, out.dtype, extra_tol)
    excess = diff - tol
    worst = float(excess.max()) if o.size else -1.0
    print("forward: flat max abs error %.4g" % err)
    assert worst <= 0, "forward error exceeds tolerance by %.4g (max abs error %.4g)" % (worst, err)
    if activation == "softmax":
        l = lse.cpu().numpy().astype(np.float64)
        if q_rows is not None:
            l = l[:, q_rows]
        ninf = np.isneginf(ref_lse)
        assert np.array_equal(np.isneginf(l), ninf), "lse -inf pattern differs"
        if (~ninf).any():
            tol = LSE_ATOL if lse_atol is None else np.broadcast_to(lse_atol, ref_lse.shape)[~ninf]
            diff = np.abs(l[~ninf] - ref_lse[~ninf])
            lerr = float(diff.max())
            print("lse: max abs error %.4g" % lerr)
            assert np.all(diff <= tol), "lse abs error %.4g exceeds its bound by %.4g" % (lerr, float(np.max(diff - tol)))
    return err


def rel_l2(a, r):
    nr = np.linalg.norm(r)
    na = np.linalg.norm(a - r)
    if nr == 0:
        return na
    return na / nr


def seq_rel_l2(a, r, offsets, mag=None):
    """Worst per-sequence relative L2 error of a jagged gradient [rows, H, d]
    whose sequence b owns rows offsets[b] .. offsets[b+1]-1, each sequence's
    reference norm floored at SEQ_NORM_FLOOR of its size's share of the
    whole tensor's norm, and (mag given: the gradient's term magnitudes,
    grad_term_magnitudes) at MAG_FLOOR of the norm of its own term
    magnitudes; and the sequence it occurs in.  A tensor that is zero in
    exact arithmetic everywhere (e.g. dq and dk when every visible query
    sees a single key: dP = delta, so dS = 0) has no scale to be relative
    to: as rel_l2 does for a zero tensor, the error is then the absolute
    norm (the magnitudes of its few terms -- one query against one key --
    can be small against what fp32 leaves of them, which is itself small in
    absolute terms)."""
    n = a.shape[0]
    tot = np.linalg.norm(r)
    worst, at = 0.0, -1
    for b in range(len(offsets) - 1):
        s0, s1 = int(offsets[b]), int(offsets[b + 1])
        if s1 <= s0:
            continue
        rb = r[s0:s1]
        den = max(np.linalg.norm(rb), SEQ_NORM_FLOOR * tot * math.sqrt((s1 - s0) / n))
        if mag is not None and tot > 0:
            den = max(den, MAG_FLOOR * np.linalg.norm(mag[s0:s1]))
        err = np.linalg.norm(a[s0:s1] - rb)
        e = float(err / den) if den > 0 else float(err)
        if e > worst:
            worst, at = e, b
    return worst, at


def beyond_slack(got, ref, allowance):
    """got with each element's difference from ref reduced by its allowance
    (to zero where the difference is within it)."""
    d = got - ref
    return ref + np.sign(d) * np.maximum(np.abs(d) - allowance, 0.0)


def check_backward(grads, refs, q_rows=None, k_rows=None, q_off=None, k_off=None, mags=None):
    """Gates dq, dk, dv: relative L2 error per tensor, and per sequence when
    the offsets of the compared rows are given (q_off for dq, k_off for dk and
    dv: the offsets of the rows as selected by q_rows / k_rows).  mags: the
    gradients' term magnitudes (grad_term_magnitudes) like refs, for the
    per-sequence floor MAG_FLOOR."""
    errs = []
    for i, (name, g, r) in enumerate(zip(("dq", "dk", "dv"), grads, refs)):
        a = to_f64(g)
        rows = q_rows if name == "dq" else k_rows
        if rows is not None:
            a = a[rows]
        tol = GRAD_RTOL if g.dtype == torch.bfloat16 else GRAD_RTOL_FP32
        e = rel_l2(a, r)
        assert e <= tol, "%s relative L2 error %.4g > %g" % (name, e, tol)
        off = q_off if name == "dq" else k_off
        if off is not None:
            ws, at = seq_rel_l2(a, r, off, None if mags is None else mags[i])
            print("%s: relative L2 %.4g, worst sequence %.4g (sequence %d)" % (name, e, ws, at))
            assert ws <= tol, "%s relative L2 error %.4g in sequence %d > %g" % (name, ws, at, tol)
        errs.append(e)
    return errs


def grad_term_magnitudes(q, k, v, dout, q_offsets, kv_offsets, scale, activation, causal):
    """Per-element sums of the magnitudes of the terms each gradient element
    is made of (dq, dk, dv like q, k, v; float64 [T, H, d]; sequence b owns
    rows q_offsets[b] .. and kv_offsets[b] ..), with softmax's
    dS = P dP - P delta taken as its two parts:
      softmax  dV_j: sum_i P_ij |dO_i|;
               dK_j: scale sum_i P_ij (|dP_ij| + |delta_i|) |q_i|,
               dQ_i: scale sum_j P_ij (|dP_ij| + |delta_i|) |k_j|;
      SiLU     dV_j: sum_i |w_ij| |dO_i|, w = silu(scale q.k) / L_kv;
               dK_j, dQ_i: scale sum |silu'(scale q.k)| |dP| / L_kv |q_i| (|k_j|).
    fp32 arithmetic leaves a residue of a small multiple of u = 2^-24 times
    these, whatever the exact value: where the terms cancel (one key: dP =
    delta, so dS = 0 and dK = dQ = 0) the residue is all the fp32 result is,
    and it has no scale of its own to be relative to."""
    from oracle.attention import visible_mask
    mq, mk, mv = np.zeros(q.shape), np.zeros(k.shape), np.zeros(v.shape)
    for b in range(len(q_offsets) - 1):
        q0, q1, k0, k1 = int(q_offsets[b]), int(q_offsets[b + 1]), int(kv_offsets[b]), int(kv_offsets[b + 1])
        lq, lk = q1 - q0, k1 - k0
        if lq == 0 or lk == 0:
            continue
        vis = visible_mask(lq, lk, causal)
        for h in range(q.shape[1]):
            qs, ks, vs, dos = q[q0:q1, h], k[k0:k1, h], v[k0:k1, h], dout[q0:q1, h]
            x = scale * (qs @ ks.T)
            dp = np.abs(dos @ vs.T)
            if activation == "softmax":
                xm = np.where(vis, x, -np.inf)
                m = np.max(xm, axis=1, keepdims=True)
                e = np.where(vis, np.exp(xm - np.where(np.isfinite(m), m, 0.0)), 0.0)
                den = e.sum(axis=1, keepdims=True)
                w = e / np.where(den > 0, den, 1.0)
                delta = np.abs(((w @ vs) * dos).sum(axis=1, keepdims=True))
                t = w * (dp + delta)
            else:
                sg = 1.0 / (1.0 + np.exp(-x))
                w = np.where(vis, np.abs(x * sg) / lk, 0.0)
                t = np.where(vis, np.abs(sg * (1.0 + x * (1.0 - sg))) / lk, 0.0) * dp
            mv[k0:k1, h] = w.T @ np.abs(dos)
            mk[k0:k1, h] = scale * (t.T @ np.abs(qs))
            mq[q0:q1, h] = scale * (t @ np.abs(ks))
    return mq, mk, mv


def grad_term_magnitudes_of(batch):
    """grad_term_magnitudes for a jagged batch as the jagged calls take it."""
    return grad_term_magnitudes(batch.f64("q"), batch.f64("k"), batch.f64("v"), batch.f64("dout"), batch.q_offsets,
                                batch.kv_offsets, batch.scale, batch.workload.activation, batch.workload.causal)


def seq_offsets(batch, seqs=None):
    """(q offsets, kv offsets) of the rows the oracle helpers return: the
    batch's own, or those of the subset `seqs` in order."""
    if seqs is None:
        return batch.q_offsets, batch.kv_offsets
    qo, ko = batch.q_offsets, batch.kv_offsets
    return (offsets_from_lengths([qo[b + 1] - qo[b] for b in seqs]),
            offsets_from_lengths([ko[b + 1] - ko[b] for b in seqs]))
