"""MXFP8 backward on the GPU against the oracle (oracle.mx.mx_attention_bwd).

Inputs: bf16 q, k, v and dout; out and lse are the oracle's MXFP8 forward of
the same q, k, v, rounded to bf16 and fp32, so that both sides start from
the same values (nothing the kernel computed goes into the reference).

Gates (tests.mx_util.MX_GRAD_RTOL per tensor, MX_GRAD_SEQ_RTOL per
sequence): relative L2 error of dq, dk and dv against the oracle's gradients
rounded to bf16, each element's difference first reduced by the allowance of
tests.mx_util.bwd_slack.  The kernel and the oracle quantise the same values
by the same rules, so what separates them is fp32 against fp64 arithmetic:
an E4M3 decision of P or dS that fp32 takes the other way near a boundary
(the allowance bounds its effect, element by element), or a bf16 rounding.
The quantisation itself moves the gradients by 6 to 9 % (relative L2), and
the plausible mistakes of a kernel -- blocks not counted from the
sequence's start, row images where column images belong, P or dS left
unquantised -- by 1 % or more, which test_mx_bwd_gates_separate_mistakes
(tests/test_oracle_mx.py) checks on the CPU with the allowance taken off.
"""

import dataclasses

import numpy as np
import pytest
import torch

import oracle.mx as mx
from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch, to_bf16_bits
from tests.gpu_util import beyond_slack, dev, rel_l2, rows_of, seq_rel_l2, to_f64, values_to_device
from tests.mx_util import MX_GRAD_RTOL, MX_GRAD_SEQ_RTOL, bwd_slack

pytestmark = pytest.mark.gpu


CASES = {
    # name: (head_dim, heads, q lengths, kv lengths, causal)
    "self_causal_d128": (128, 2, [1, 31, 32, 33, 64, 65, 200, 130], None, True),
    "self_noncausal_d64": (64, 3, [7, 64, 129, 300], None, False),
    "cross_d64": (64, 2, [1, 17, 64, 130], [300, 5, 64, 1000], False),
    "cross_causal_d128": (128, 1, [100, 40, 3], [30, 70, 200], True),
    "empty_sequences": (128, 2, [0, 5, 3, 0, 70], [7, 0, 40, 0, 70], True),
    "long_d128": (128, 1, [700, 129], [1030, 129], False),
    "many_heads": (64, 16, [50, 2], None, True),
}


def _case(name, seed):
    d, H, lq, lk, causal = CASES[name]
    lk = lq if lk is None else lk
    wl = dataclasses.replace(WORKLOADS["selfattn_causal"], head_dim=d, heads=H, causal=causal)
    return make_batch(wl, seed, q_lengths=lq, kv_lengths=lk, with_dout=True)


def _bf16_round(x):
    """float64 -> the float64 value of its bf16 rounding (nearest even)."""
    bits = to_bf16_bits(np.asarray(x, dtype=np.float32)).astype(np.uint32) << 16
    return bits.view(np.float32).astype(np.float64)


def _oracle_inputs(b, seqs=None):
    """The oracle's MXFP8 forward of the batch (or of the sequences in
    `seqs` alone, sequences being independent): out rounded to bf16, lse to
    fp32, -inf kept."""
    q, k, v = b.f64("q"), b.f64("k"), b.f64("v")
    qo, ko = b.q_offsets, b.kv_offsets
    if seqs is not None:
        qr, kr = rows_of(b, seqs, "q"), rows_of(b, seqs, "k")
        q, k, v = q[qr], k[kr], v[kr]
        qo = np.concatenate([[0], np.cumsum(b.q_lengths[seqs])])
        ko = np.concatenate([[0], np.cumsum(b.kv_lengths[seqs])])
    out, lse = mx.mx_attention_fwd(q, k, v, qo, ko, b.scale, b.workload.causal)
    return _bf16_round(out), lse.astype(np.float32).astype(np.float64)


def _device_case(b, out64, lse64):
    q, k, v, do = (values_to_device(x, "bf16") for x in (b.q, b.k, b.v, b.dout))
    out = values_to_device(to_bf16_bits(np.asarray(out64, dtype=np.float32)), "bf16")
    lse = torch.from_numpy(np.ascontiguousarray(lse64, dtype=np.float32)).to(dev())
    qo = torch.from_numpy(b.q_offsets.astype(np.int32)).to(dev())
    ko = torch.from_numpy(b.kv_offsets.astype(np.int32)).to(dev())
    mq = int(b.q_lengths.max()) if len(b.q_lengths) else 0
    mk = int(b.kv_lengths.max()) if len(b.kv_lengths) else 0
    return q, k, v, out, do, lse, qo, ko, mq, mk


def _reference(*args):
    """The oracle's gradients for mx_attention_bwd's arguments, and the
    allowance (tests.mx_util.bwd_slack) for the E4M3 decisions of P and dS
    that fp32 may take the other way."""
    return mx.mx_attention_bwd(*args), bwd_slack(*args)


def _check(got, ref, q_offsets, kv_offsets, label, slack=None):
    """got: (dq, dk, dv) device bf16; ref: oracle (dq, dk, dv) float64;
    slack: per-element allowances like ref, taken off |got - ref| first."""
    slack = (0.0, 0.0, 0.0) if slack is None else slack
    for name, g, r, off, a in zip(("dq", "dk", "dv"), got, ref, (q_offsets, kv_offsets, kv_offsets), slack):
        a = np.broadcast_to(a, r.shape)
        g = to_f64(g)
        r = _bf16_round(r)
        assert np.all(np.isfinite(g)), "%s %s: non-finite values" % (label, name)
        raw = rel_l2(g, r)
        g = beyond_slack(g, r, a)
        e = rel_l2(g, r)
        ws, at = seq_rel_l2(g, r, off)
        print("%s %s: rel L2 %.3g (%.3g before the allowance), worst sequence %.3g (sequence %d)"
              % (label, name, e, raw, ws, at))
        assert e <= MX_GRAD_RTOL, "%s %s: rel L2 %.4g" % (label, name, e)
        assert ws <= MX_GRAD_SEQ_RTOL, "%s %s: sequence %d rel L2 %.4g" % (label, name, at, ws)


@pytest.mark.parametrize("name", sorted(CASES))
def test_mx_backward_parity(name):
    b = _case(name, 2000 + sorted(CASES).index(name))
    print("case", name, flush=True)
    out64, lse64 = _oracle_inputs(b)
    q, k, v, out, do, lse, qo, ko, mq, mk = _device_case(b, out64, lse64)
    got = jfa.mx_backward(q, k, v, out, do, lse, qo, ko, mq, mk, b.scale, b.workload.causal)
    torch.cuda.synchronize()
    ref, slack = _reference(b.f64("q"), b.f64("k"), b.f64("v"), out64, b.f64("dout"), lse64, b.q_offsets,
                            b.kv_offsets, b.scale, b.workload.causal)
    _check(got, ref, b.q_offsets, b.kv_offsets, name, slack)
    # rows of sequences without keys (dq) or queries (dk, dv) are zero
    for g, lens_other, off in ((got[0], b.kv_lengths, b.q_offsets), (got[1], b.q_lengths, b.kv_offsets),
                               (got[2], b.q_lengths, b.kv_offsets)):
        for s in np.nonzero(lens_other == 0)[0]:
            assert not (g[int(off[s]):int(off[s + 1])] != 0).any()


@pytest.mark.parametrize("name", ["mx_selfattn_causal", "mx_cross_asym"])
def test_mx_backward_full_size_sampled(name):
    """Full-size batches as the benchmark runs them; the oracle computes the
    forward and backward of sampled sequences alone (the other sequences get
    zero out and lse, which changes nothing for the sampled ones)."""
    b = make_batch(name, 9, with_dout=True)
    rng = np.random.default_rng(9)
    lens = b.q_lengths * np.maximum(b.kv_lengths, 1)
    seqs = sorted({int(np.argmax(lens))} | set(int(x) for x in rng.choice(len(lens), 3, replace=False)))
    out_s, lse_s = _oracle_inputs(b, seqs)
    qr, kr = rows_of(b, seqs, "q"), rows_of(b, seqs, "k")
    H = b.workload.heads
    out64 = np.zeros((len(b.q), H, b.workload.head_dim))
    lse64 = np.zeros((H, len(b.q)))
    out64[qr] = out_s
    lse64[:, qr] = lse_s
    q, k, v, out, do, lse, qo, ko, mq, mk = _device_case(b, out64, lse64)
    got = jfa.mx_backward(q, k, v, out, do, lse, qo, ko, mq, mk, b.scale, b.workload.causal)
    torch.cuda.synchronize()
    for g in got:
        assert torch.isfinite(g).all()
    qs = np.concatenate([[0], np.cumsum(b.q_lengths[seqs])])
    ks = np.concatenate([[0], np.cumsum(b.kv_lengths[seqs])])
    ref, slack = _reference(b.f64("q")[qr], b.f64("k")[kr], b.f64("v")[kr], out_s, b.f64("dout")[qr], lse_s, qs,
                            ks, b.scale, b.workload.causal)
    _check((got[0][torch.from_numpy(qr).to(dev())], got[1][torch.from_numpy(kr).to(dev())],
            got[2][torch.from_numpy(kr).to(dev())]), ref, qs, ks, name, slack)


def test_mx_backward_images_equals_backward_and_is_reproducible():
    """jfa_mx_backward is jfa_mx_quantize of the seven operands followed by
    jfa_mx_backward_images, bit for bit; and two calls agree bit for bit."""
    b = _case("cross_causal_d128", 78)
    out64, lse64 = _oracle_inputs(b)
    q, k, v, out, do, lse, qo, ko, mq, mk = _device_case(b, out64, lse64)
    wl = b.workload
    g1 = jfa.mx_backward(q, k, v, out, do, lse, qo, ko, mq, mk, b.scale, wl.causal)
    g2 = jfa.mx_backward(q, k, v, out, do, lse, qo, ko, mq, mk, b.scale, wl.causal)
    src = {"q": (q, qo), "k": (k, ko), "v": (v, ko), "dout": (do, qo)}
    images = [jfa.mx_quantize(src[t][0], src[t][1], lay) for t, lay in jfa.MX_BACKWARD_IMAGES]
    g3 = jfa.mx_backward_images(images, out, do, lse, qo, ko, wl.heads, wl.head_dim, q.shape[0], k.shape[0], mq, mk,
                                b.scale, wl.causal)
    torch.cuda.synchronize()
    for a, c, e in zip(g1, g2, g3):
        assert torch.equal(a.view(torch.int16), c.view(torch.int16))
        assert torch.equal(a.view(torch.int16), e.view(torch.int16))
