"""MXFP8 path on the GPU against the oracle (oracle.mx):

* the quantisation kernel's images, bit for bit (codes and scale codes);
* the attention forward, element by element, within the bf16 forward bound
  plus the allowance for weights whose fp64 value sits on a rounding or floor
  boundary (tests.mx_util.fwd_slack; there the kernel's fp32 decision and the
  oracle's may differ and both are correct);
* inputs on which MXFP8 is lossless, against exact attention;
* full-size batches, sampled sequences.
"""

import dataclasses
import math

import numpy as np
import pytest
import torch

import oracle
import oracle.mx as mx
from jagged_attention_ads_amd import jfa
from jagged_attention_ads_amd.workloads import WORKLOADS, make_batch, to_bf16_bits
from tests import mx_util
from tests.gpu_util import LSE_ATOL, dev, forward_tolerance, rows_of, to_f64, values_to_device

pytestmark = pytest.mark.gpu


def _offsets_dev(lengths):
    off = np.concatenate([[0], np.cumsum(lengths)]).astype(np.int32)
    return off, torch.from_numpy(off).to(dev())


def _bf16(x):
    """float64 values -> (bf16 device tensor, the exact float64 values it holds)."""
    bits = to_bf16_bits(np.asarray(x, dtype=np.float32))
    t = values_to_device(bits, "bf16")
    return t, to_f64(t)


def _special_values(rng, T, H, d):
    """Normal values with whole blocks of zeros, of tiny values (scale code
    0), of large values, a negative zero and exact ties after scaling."""
    x = rng.standard_normal((T, H, d)) * np.exp2(rng.integers(-4, 5, (T, H, 1)))
    if T > 3:
        x[0, 0, :32] = 0.0
        x[1, 0, :32] = rng.standard_normal(32) * 2.0 ** -125
        x[2, 0, :] = rng.standard_normal(d) * 2.0 ** 100
        x[3, 0, 5] = -0.0
        # block max 1 -> scale 2^-8: 1.0625 * 2^-8 * 256 = ... elements 272 = midpoint of 256 and 288
        x[3, 0, 32:64] = 0.5
        x[3, 0, 32] = 1.0
        x[3, 0, 33] = 272.0 / 256.0
        x[3, 0, 34] = 304.0 / 256.0
    return x


@pytest.mark.parametrize("d", [64, 128])
@pytest.mark.parametrize("layout", ["rows", "keys"])
def test_quantize_bit_exact(d, layout):
    rng = np.random.default_rng(40 + d + (layout == "keys"))
    lengths = [5, 0, 64, 33, 100, 1, 31]
    off, offd = _offsets_dev(lengths)
    H = 3
    xd, x = _bf16(_special_values(rng, int(off[-1]), H, d))
    img = jfa.mx_quantize(xd, offd, layout).cpu().numpy()
    if layout == "rows":
        codes, scales = mx_util.decode_rows_image(img, off, H, d)
        want_c, want_e = mx.mx_quantize_rows(x)
        assert np.array_equal(codes, want_c)
        assert np.array_equal(scales.astype(np.int64), want_e + 127)
    else:
        codes, scales, tail = mx_util.decode_keys_image(img, off, H, d)
        want_c, want_e = mx.mx_quantize_keys(x, off)
        assert np.array_equal(codes, want_c)
        assert np.array_equal(scales.astype(np.int64), want_e + 127)
        assert not tail.any()


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
    return make_batch(wl, seed, q_lengths=lq, kv_lengths=lk, with_dout=False)


def _run(b):
    wl = b.workload
    q = values_to_device(b.q, "bf16")
    k = values_to_device(b.k, "bf16")
    v = values_to_device(b.v, "bf16")
    qo = torch.from_numpy(b.q_offsets.astype(np.int32)).to(dev())
    ko = torch.from_numpy(b.kv_offsets.astype(np.int32)).to(dev())
    mq = int(b.q_lengths.max()) if len(b.q_lengths) else 0
    mk = int(b.kv_lengths.max()) if len(b.kv_lengths) else 0
    out, lse = jfa.mx_forward(q, k, v, qo, ko, mq, mk, b.scale, wl.causal)
    torch.cuda.synchronize()
    return out, lse


def _check(out, lse, q, k, v, qo, ko, scale, causal, q_rows=None):
    ref, ref_lse = mx.mx_attention_fwd(q, k, v, qo, ko, scale, causal)
    slack = mx_util.fwd_slack(q, k, v, qo, ko, scale, causal)
    got = to_f64(out)
    gl = lse.double().cpu().numpy()
    if q_rows is not None:
        got, gl = got[q_rows], gl[:, q_rows]
    tol = forward_tolerance(ref, torch.bfloat16) + slack
    err = np.abs(got - ref)
    print("mx forward: max abs err %.3g, max err beyond the flat bound %.3g, rows with slack %d"
          % (err.max(initial=0), (err - forward_tolerance(ref, torch.bfloat16)).max(initial=0),
             int((slack.max(axis=2) > 0).sum())))
    assert np.all(err <= tol), np.unravel_index(np.argmax(err - tol), err.shape)
    live = np.isfinite(ref_lse)
    assert np.array_equal(live, np.isfinite(gl))
    assert np.abs(gl[live] - ref_lse[live]).max(initial=0) <= LSE_ATOL


@pytest.mark.parametrize("name", sorted(CASES))
def test_mx_forward_parity(name):
    b = _case(name, 1000 + sorted(CASES).index(name))
    print("case", name, flush=True)
    out, lse = _run(b)
    _check(out, lse, b.f64("q"), b.f64("k"), b.f64("v"), b.q_offsets, b.kv_offsets, b.scale, b.workload.causal)


@pytest.mark.parametrize("causal", [False, True])
@pytest.mark.parametrize("d", [64, 128])
def test_mx_forward_lossless_equals_exact_attention(causal, d):
    """Integer scores (scale ln 2: t = q.k), small enough spreads and exactly
    representable operands: every quantisation is exact, so MXFP8 attention
    is exact attention."""
    from tests.test_oracle_mx import _lossless_inputs
    lq = [1, 40, 0, 70, 33, 130]
    lk = [1, 40, 5, 100, 65, 130] if not causal else [1, 40, 5, 70, 65, 130]
    q, k, v, qo, ko = _lossless_inputs(lq, lk, 2, d, seed=5 + d)
    qd, _ = _bf16(q)
    kd, _ = _bf16(k)
    vd, _ = _bf16(v)
    qod = torch.from_numpy(qo.astype(np.int32)).to(dev())
    kod = torch.from_numpy(ko.astype(np.int32)).to(dev())
    out, lse = jfa.mx_forward(qd, kd, vd, qod, kod, max(lq), max(lk), math.log(2.0), causal)
    torch.cuda.synchronize()
    ref, ref_lse = oracle.attention_fwd(q, k, v, qo, ko, math.log(2.0), "softmax", causal)
    got = to_f64(out)
    assert np.all(np.abs(got - ref) <= forward_tolerance(ref, torch.bfloat16))
    gl = lse.double().cpu().numpy()
    live = np.isfinite(ref_lse)
    assert np.array_equal(live, np.isfinite(gl))
    assert np.abs(gl[live] - ref_lse[live]).max(initial=0) <= LSE_ATOL


@pytest.mark.parametrize("name", ["selfattn_causal", "cross_asym"])
def test_mx_full_size_sampled(name):
    """Full-size batches, as the benchmark runs them; the oracle recomputes
    sampled sequences alone (sequences are independent)."""
    b = make_batch(name, 7, with_dout=False)
    out, lse = _run(b)
    assert torch.isfinite(out).all()
    rng = np.random.default_rng(7)
    lens = b.q_lengths * np.maximum(b.kv_lengths, 1)
    seqs = sorted({int(np.argmax(lens))} | set(int(x) for x in rng.choice(len(lens), 3, replace=False)))
    qr, kr = rows_of(b, seqs, "q"), rows_of(b, seqs, "k")
    qs = np.concatenate([[0], np.cumsum(b.q_lengths[seqs])])
    ks = np.concatenate([[0], np.cumsum(b.kv_lengths[seqs])])
    _check(out, lse, b.f64("q")[qr], b.f64("k")[kr], b.f64("v")[kr], qs, ks, b.scale, b.workload.causal,
           q_rows=qr)


SHORT_Q = {
    # name: (head_dim, heads, q lengths (each at most 64), kv lengths, causal)
    "short_q_d64": (64, 8, [1, 17, 64, 0, 33, 5], [300, 5, 1000, 40, 0, 129], False),
    "short_q_causal_d128": (128, 2, [64, 1, 40, 63], [64, 700, 33, 2], True),
}


@pytest.mark.parametrize("name", sorted(SHORT_Q))
def test_mx_two_wave_forward(name, options):
    """No sequence longer than 64 queries: the forward runs two waves per
    item.  Its outputs equal the four-wave kernel's (JFA_OPT_FWD_SHORT = 0)
    bit for bit, and the oracle's within the bound."""
    d, H, lq, lk, causal = SHORT_Q[name]
    wl = dataclasses.replace(WORKLOADS["selfattn_causal"], head_dim=d, heads=H, causal=causal)
    b = make_batch(wl, 1300 + sorted(SHORT_Q).index(name), q_lengths=lq, kv_lengths=lk, with_dout=False)
    print("case", name, flush=True)
    out, lse = _run(b)
    options("fwd_short", 0)
    out4, lse4 = _run(b)
    assert torch.equal(out.view(torch.int16), out4.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse4.view(torch.int32))
    _check(out, lse, b.f64("q"), b.f64("k"), b.f64("v"), b.q_offsets, b.kv_offsets, b.scale, causal)


def test_mx_attend_from_images_equals_forward():
    """jfa_mx_forward is jfa_mx_quantize of q, k, v then jfa_mx_attend, bit
    for bit."""
    b = _case("cross_causal_d128", 77)
    wl = b.workload
    q, k, v = (values_to_device(x, "bf16") for x in (b.q, b.k, b.v))
    qo = torch.from_numpy(b.q_offsets.astype(np.int32)).to(dev())
    ko = torch.from_numpy(b.kv_offsets.astype(np.int32)).to(dev())
    mq, mk = int(b.q_lengths.max()), int(b.kv_lengths.max())
    out, lse = jfa.mx_forward(q, k, v, qo, ko, mq, mk, b.scale, wl.causal)
    qi, ki, vi = jfa.mx_quantize(q, qo, "rows"), jfa.mx_quantize(k, ko, "rows"), jfa.mx_quantize(v, ko, "keys")
    out2, lse2 = jfa.mx_attend(qi, ki, vi, qo, ko, wl.heads, wl.head_dim, q.shape[0], k.shape[0], mq, mk, b.scale,
                               wl.causal)
    torch.cuda.synchronize()
    assert torch.equal(out.view(torch.int16), out2.view(torch.int16))
    assert torch.equal(lse.view(torch.int32), lse2.view(torch.int32))
