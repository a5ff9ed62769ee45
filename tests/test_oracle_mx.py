"""Pins of the MXFP8 oracle (oracle.mx) against what the OCP MX format and the
mathematics fix: the E4M3 table values, brute-force nearest-value rounding,
closed-form block exponents and error bounds, hand-worked quantisations of the
softmax numerator (tests/golden/mx_cases.json), lossless cases in which MXFP8
attention must equal the exact attention oracle, and an independent per-element
loop implementation on tiny inputs.
"""

import json
import math
import os

import numpy as np
import pytest

import oracle
import oracle.mx as mx

GOLDEN = os.path.join(os.path.dirname(__file__), "golden", "mx_cases.json")
CASES = json.load(open(GOLDEN))

# every finite E4M3 value, by code (brute-force reference for rounding)
FINITE = np.array([c for c in range(256) if c not in (0x7F, 0xFF)])


def _table_value(c):
    """E4M3 value from the bit fields, written out per code (no vector code
    shared with the oracle)."""
    s = -1.0 if c & 0x80 else 1.0
    e = (c >> 3) & 15
    m = c & 7
    if e == 0:
        return s * m * 2.0 ** -9
    return s * (8 + m) * 2.0 ** (e - 10)


TABLE = np.array([_table_value(c) for c in FINITE])


def _nearest_code(x):
    """Brute force: the finite code nearest to x after clamping to +-448, ties
    to the code with even mantissa; zero keeps the sign of x."""
    a = min(abs(x), 448.0)
    pos = FINITE[(FINITE & 0x80) == 0]
    vals = TABLE[(FINITE & 0x80) == 0]
    d = np.abs(vals - a)
    best = np.nonzero(d == d.min())[0]
    c = int(pos[best[0]]) if len(best) == 1 else int([pos[i] for i in best if pos[i] % 2 == 0][0])
    return c | (0x80 if math.copysign(1.0, x) < 0 else 0)


# ------------------------------------------------------------------ E4M3


def test_e4m3_table_values():
    for e in CASES["e4m3"]:
        assert mx.e4m3_decode(e["code"]) == e["value"], e["what"]
        assert int(mx.e4m3_encode(e["value"])) == e["code"], e["what"]
    for c in CASES["e4m3_nan"]:
        assert np.isnan(mx.e4m3_decode(c))


def test_e4m3_decode_matches_bit_fields():
    assert np.array_equal(mx.e4m3_decode(FINITE), TABLE)


def test_e4m3_round_trip():
    vals = mx.e4m3_decode(FINITE)
    codes = mx.e4m3_encode(vals)
    # +0 and -0 keep their own codes
    assert np.array_equal(codes.astype(int), FINITE)


def test_e4m3_encode_brute_force():
    rng = np.random.default_rng(3)
    x = rng.choice([-1, 1], 4000) * np.exp2(rng.uniform(-12, 9.6, 4000))
    x = np.concatenate([x, [0.0, -0.0, 448.0, 463.9, 464.0, 470.0, 1e6, -1e6, 2.0 ** -10, 3 * 2.0 ** -11]])
    got = mx.e4m3_encode(x)
    want = np.array([_nearest_code(v) for v in x])
    assert np.array_equal(got.astype(int), want)


def test_e4m3_ties_go_to_even_mantissa():
    pos = np.sort(TABLE[(FINITE & 0x80) == 0])
    mids = (pos[:-1] + pos[1:]) / 2
    codes = mx.e4m3_encode(mids).astype(int)
    assert np.all(codes % 2 == 0)
    # and a hair off the midpoint goes to the nearer neighbour
    up = mx.e4m3_encode(mids * (1 + 1e-9)).astype(int)
    assert np.array_equal(mx.e4m3_decode(up), pos[1:])


def test_e4m3_saturates_instead_of_nan():
    assert int(mx.e4m3_encode(500.0)) == 0x7E
    assert int(mx.e4m3_encode(-1e30)) == 0xFE


# ------------------------------------------------------------------ MX blocks


@pytest.mark.parametrize("k", [-120, -10, -1, 0, 3, 20])
def test_block_exponent_closed_form(k):
    for f in (1.0, 1.25, 1.999999):
        assert int(mx.e8m0_exponent(f * 2.0 ** k)) == max(k - 8, -127)


def test_block_saturation_of_a_large_block_max():
    # max in (1.75, 2) * 2^k: scale 2^(k-8), the max itself clamps to 448
    codes, ex = mx.mx_quantize_block(np.array([1.875, 1.0]))
    assert ex == -8 and codes.tolist() == [0x7E, 0x78]


def test_block_exponent_clamps():
    assert int(mx.e8m0_exponent(0.0)) == -127
    assert int(mx.e8m0_exponent(2.0 ** -130)) == -127
    assert int(mx.e8m0_exponent(2.0 ** 200)) == 127


def test_block_error_bound():
    rng = np.random.default_rng(5)
    for _ in range(200):
        v = rng.standard_normal(32) * np.exp2(rng.uniform(-20, 20))
        codes, ex = mx.mx_quantize_block(v)
        X = 2.0 ** ex
        deq = mx.e4m3_decode(codes) * X
        a = np.abs(v) / X
        assert a.max() < 512
        # normal range: half a spacing of the element's binade; subnormal
        # range: half of 2^-9; beyond 448: clamped
        half = np.where(a >= 2.0 ** -6, np.exp2(np.floor(np.log2(np.maximum(a, 2.0 ** -6))) - 4), 2.0 ** -10)
        sat = a > 448
        assert np.all(np.abs(deq - v)[~sat] <= half[~sat] * X * (1 + 1e-12))
        assert np.all(np.abs(deq[sat]) == 448 * X)


def test_rows_lossless_when_representable():
    rng = np.random.default_rng(6)
    # multiples of 2^-3 up to 1.75 and a block max of 1.75: every element /
    # 2^-8 is an E4M3 value (a block max in (1.75, 2) would saturate)
    x = rng.integers(-14, 15, (7, 2, 64)) * 2.0 ** -3
    x[..., 0] = 1.75
    x[..., 32] = 1.75
    codes, ex = mx.mx_quantize_rows(x)
    assert np.all(ex == -8)
    assert np.array_equal(mx.mx_dequantize_rows(codes, ex), x)


def test_keys_blocks_start_at_each_sequence():
    # sequences of 5 and 40 rows: rows 5..36 form one block, 37..44 another
    x = np.ones((45, 1, 32))
    x[36, 0, 3] = 100.0    # raises the scale of the first block of sequence 1 only
    codes, ex = mx.mx_quantize_keys(x, [0, 5, 45])
    assert np.all(ex[0:5, 0, :] == -8)
    assert np.all(ex[5:37, 0, 3] == 6 - 8) and np.all(ex[5:37, 0, 4] == -8)
    assert np.all(ex[37:45, 0, :] == -8)
    assert np.array_equal(mx.mx_dequantize_keys(codes, ex)[37:], x[37:])


# ------------------------------------------------------------------ online P


@pytest.mark.parametrize("case", range(3))
def test_p_quantisation_worked_examples(case):
    e = CASES["p_examples"][case]
    t = np.array(e["t"])
    n = len(t)
    codes, fb = mx.quantize_p(t[None, :], np.ones((1, n), bool))
    assert codes[0].tolist() == e["codes"], e["derivation"]
    # the same through the attention: scale ln 2 makes t = q.k
    q = np.zeros((1, 1, 32))
    q[0, 0, 0] = 1.0
    k = np.zeros((n, 1, 32))
    k[:, 0, 0] = t
    v = np.zeros((n, 1, 32))
    for j in range(n):
        v[j, 0, j] = 1.0
    out, lse = mx.mx_attention_fwd(q, k, v, [0, 1], [0, n], math.log(2.0))
    np.testing.assert_allclose(out[0, 0, :n], e["out"], rtol=1e-12, atol=0)
    assert np.all(out[0, 0, n:] == 0)
    np.testing.assert_allclose(lse[0, 0], e["lse"], rtol=1e-12)


def _lossless_inputs(lq, lk, heads, d, seed):
    """Q, K with small integer q.k (scale ln 2 then makes every t an integer, so
    every P element is an exact power of two) and V exactly
    representable: MXFP8 attention then equals exact attention."""
    rng = np.random.default_rng(seed)
    qo = np.concatenate([[0], np.cumsum(lq)])
    ko = np.concatenate([[0], np.cumsum(lk)])
    # at most 6 entries +-1 per row of q besides the 2s below: |q.k| <= 6 + 2 d/32,
    # so the elements 2^(t - floor(max) + 8) of a block stay above 2^-9
    q = np.zeros((qo[-1], heads, d))
    for r in range(qo[-1]):
        for h in range(heads):
            cols = rng.choice([c for c in range(d) if c % 32], 6, replace=False)
            q[r, h, cols] = rng.choice([-1.0, 1.0], 6)
    k = rng.integers(-1, 2, (ko[-1], heads, d)).astype(np.float64)
    v = rng.integers(-14, 15, (ko[-1], heads, d)) * 2.0 ** -3
    # every column block of V (32 keys of a sequence) holds a 1.75 somewhere,
    # so its scale is 2^-8 and every element is exact
    for b in range(len(lk)):
        for r0 in range(int(ko[b]), int(ko[b + 1]), 32):
            v[r0] = 1.75
    # row blocks of Q and K hold a 2 (resp. 1): scales 2^-7 / 2^-8, exact
    q[..., ::32] = 2.0
    k[..., ::32] = 1.0
    return q, k, v, qo, ko


@pytest.mark.parametrize("causal", [False, True])
def test_attention_equals_exact_attention_when_lossless(causal):
    lq, lk = [1, 40, 0, 70, 33], [1, 40, 5, 100, 65]
    q, k, v, qo, ko = _lossless_inputs(lq, lk, 2, 64, seed=11)
    out, lse = mx.mx_attention_fwd(q, k, v, qo, ko, math.log(2.0), causal)
    ref, ref_lse = oracle.attention_fwd(q, k, v, qo, ko, math.log(2.0), "softmax", causal)
    np.testing.assert_allclose(out, ref, rtol=1e-12, atol=1e-12)
    live = np.isfinite(ref_lse)
    assert np.array_equal(live, np.isfinite(lse))
    np.testing.assert_allclose(lse[live], ref_lse[live], rtol=1e-12, atol=1e-12)


def test_attention_uniform_scores_average_quantised_v():
    rng = np.random.default_rng(2)
    lq, lk = [3, 50], [7, 90]
    qo = np.array([0, 3, 53])
    ko = np.array([0, 7, 97])
    q = np.zeros((53, 1, 32))
    k = rng.standard_normal((97, 1, 32))
    v = rng.standard_normal((97, 1, 32))
    out, lse = mx.mx_attention_fwd(q, k, v, qo, ko, 0.3, causal=False)
    vh = mx.mx_dequantize_keys(*mx.mx_quantize_keys(v, ko))
    np.testing.assert_allclose(out[:3, 0], np.broadcast_to(vh[:7, 0].mean(0), (3, 32)), atol=1e-13)
    np.testing.assert_allclose(out[3:, 0], np.broadcast_to(vh[7:, 0].mean(0), (50, 32)), atol=1e-13)
    np.testing.assert_allclose(lse[0, :3], math.log(7), atol=1e-13)


def _loop_mx_attention(q, k, v, qo, ko, scale, causal):
    """Independent per-element implementation for tiny inputs: scalar block
    scales from the bit-level definition and brute-force rounding."""
    qh = np.zeros_like(q)
    kh = np.zeros_like(k)
    vh = np.zeros_like(v)
    T, H, d = q.shape

    def quant(vals):
        amax = max(abs(x) for x in vals)
        ex = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
        return [_table_value(_nearest_code(x / 2.0 ** ex)) * 2.0 ** ex for x in vals]

    def quant_fit(vals):   # P and dS: the least exponent whose range holds the block (R8)
        amax = max(abs(x) for x in vals)
        ex = next(e for e in range(-127, 128) if amax <= 448.0 * 2.0 ** e)
        return [_table_value(_nearest_code(x / 2.0 ** ex)) * 2.0 ** ex for x in vals]

    for r in range(T):
        for h in range(H):
            for c0 in range(0, d, 32):
                qh[r, h, c0:c0 + 32] = quant(list(q[r, h, c0:c0 + 32]))
    for r in range(k.shape[0]):
        for h in range(H):
            for c0 in range(0, d, 32):
                kh[r, h, c0:c0 + 32] = quant(list(k[r, h, c0:c0 + 32]))
    for b in range(len(ko) - 1):
        for r0 in range(ko[b], ko[b + 1], 32):
            r1 = min(r0 + 32, ko[b + 1])
            for h in range(H):
                for col in range(d):
                    vh[r0:r1, h, col] = quant(list(v[r0:r1, h, col]))
    out = np.zeros((T, H, d))
    lse = np.full((H, T), -np.inf)
    for b in range(len(qo) - 1):
        lq, lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        for i in range(lq):
            for h in range(H):
                vis = [j for j in range(lk) if not causal or j <= i + lk - lq]
                if not vis:
                    continue
                t = {j: scale / math.log(2) * float(np.dot(qh[qo[b] + i, h], kh[ko[b] + j, h])) for j in vis}
                den = sum(2.0 ** t[j] for j in vis)
                acc = np.zeros(d)
                for c in range(0, lk, 32):
                    blk = [j for j in vis if c <= j < c + 32]
                    if not blk:
                        continue
                    fb = math.floor(max(t[j] for j in blk))
                    for j in blk:
                        w = _table_value(_nearest_code(2.0 ** (t[j] - fb + 8))) * 2.0 ** (fb - 8)
                        acc += w * vh[ko[b] + j, h]
                out[qo[b] + i, h] = acc / den
                lse[h, qo[b] + i] = math.log(den)
    return out, lse


@pytest.mark.parametrize("causal", [False, True])
def test_attention_matches_loop_implementation(causal):
    rng = np.random.default_rng(17 + causal)
    lq, lk = [2, 37, 0, 5], [35, 33, 4, 0]
    qo = np.concatenate([[0], np.cumsum(lq)])
    ko = np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((qo[-1], 2, 64)) * 1.5
    k = rng.standard_normal((ko[-1], 2, 64))
    v = rng.standard_normal((ko[-1], 2, 64)) * np.exp2(rng.integers(-6, 6, (ko[-1], 2, 64)))
    out, lse = mx.mx_attention_fwd(q, k, v, qo, ko, 0.25, causal)
    ref, ref_lse = _loop_mx_attention(q, k, v, qo, ko, 0.25, causal)
    np.testing.assert_allclose(out, ref, rtol=1e-11, atol=1e-12)
    np.testing.assert_allclose(lse, ref_lse, rtol=1e-12, atol=1e-12)


def test_attention_close_to_exact_attention():
    rng = np.random.default_rng(9)
    lq, lk = [64, 130], [64, 200]
    qo = np.concatenate([[0], np.cumsum(lq)])
    ko = np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((qo[-1], 2, 128))
    k = rng.standard_normal((ko[-1], 2, 128))
    v = rng.standard_normal((ko[-1], 2, 128))
    out, lse = mx.mx_attention_fwd(q, k, v, qo, ko, 128 ** -0.5, causal=True)
    ref, ref_lse = oracle.attention_fwd(q, k, v, qo, ko, 128 ** -0.5, "softmax", True)
    # 8-bit operands: a row that sees one key returns that key's quantised V
    # row (up to 1/8 off where a block maximum saturates); on average the
    # error is about a per cent of the output scale
    assert np.abs(out - ref).max() < 0.125 * np.abs(v).max()
    assert np.abs(lse - ref_lse).max() < 0.1
    assert np.abs(out - ref).mean() < 0.015


# ------------------------------------------------------------------ backward


def _draw_bwd(lq, lk, heads, d, seed, causal):
    rng = np.random.default_rng(seed)
    qo = np.concatenate([[0], np.cumsum(lq)])
    ko = np.concatenate([[0], np.cumsum(lk)])
    q = rng.standard_normal((qo[-1], heads, d))
    k = rng.standard_normal((ko[-1], heads, d))
    v = rng.standard_normal((ko[-1], heads, d))
    do = rng.standard_normal((qo[-1], heads, d))
    out, lse = mx.mx_attention_fwd(q, k, v, qo, ko, 0.3, causal)
    return q, k, v, out, do, lse, qo, ko


@pytest.mark.parametrize("causal", [False, True])
def test_backward_without_quantisation_is_the_attention_backward(causal):
    q, k, v, _, do, _, qo, ko = _draw_bwd([3, 40, 0, 70], [35, 40, 5, 70], 2, 64, 4, causal)
    out, lse = oracle.attention_fwd(q, k, v, qo, ko, 0.3, "softmax", causal)
    got = mx.mx_attention_bwd(q, k, v, out, do, lse, qo, ko, 0.3, causal, quantize=False)
    ref = oracle.attention_bwd(q, k, v, do, qo, ko, 0.3, "softmax", causal)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-10, atol=1e-12)


def test_matrix_blocks_closed_form():
    # a 40 x 2 block: rows 0..31 and 32..39 are separate blocks per column
    x = np.ones((40, 2))
    x[5, 0] = 100.0
    y = mx.mx_quantize_matrix(x, 0)
    assert y[5, 0] == 96.0           # 100 = 1.5625 * 64 -> scale 2^-2, 400 -> nearest 384
    assert np.all(y[32:, 0] == 1.0) and np.all(y[:, 1] == 1.0)
    # along rows: the same with the matrix transposed
    np.testing.assert_array_equal(mx.mx_quantize_matrix(x.T, 1), y.T)
    # the fitted exponent (R8) where it differs from floor(log2 max) - 8: a
    # block max just below 1 keeps the scale 2^-8 (element 256 - 2^-22,
    # rounded to 256: the value 1), where the vector conversion would take
    # 2^-9 and saturate it to 448 (0.875); 1.9 takes 2^-7 (243.2 -> 240:
    # 1.875) instead of saturating to 1.75
    z = np.full((32, 3), 0.25)
    z[0] = [1.0 - 2.0 ** -30, 1.9, 1.75]
    w = mx.mx_quantize_matrix(z, 0)
    assert w[0, 0] == 1.0 and w[0, 1] == 1.875 and w[0, 2] == 1.75
    assert np.all(w[1:] == 0.25)


def test_fit_exponent_closed_forms():
    """R8: the least k with max <= 448 2^k."""
    f = mx.e8m0_exponent_fit
    assert f(1.0) == -8 and f(1.0 - 2.0 ** -40) == -8 and f(1.0 + 2.0 ** -40) == -8
    assert f(1.75) == -8 and f(1.75 * (1 + 2.0 ** -40)) == -7 and f(2.0) == -7
    assert f(448.0) == 0 and f(448.5) == 1 and f(0.0) == -127 and f(2.0 ** -200) == -127
    a = np.exp2(np.random.default_rng(2).uniform(-100, 100, 1000))
    r = a / np.exp2(f(a).astype(np.float64))
    assert np.all((r > 224.0) & (r <= 448.0))


def test_backward_lossless_values_and_uniform_weights():
    """Q = 0 makes every weight 1/L (L = 32: exact in E4M3); with V and dO
    exactly representable, dV is exact, and dK = dS^T Q = 0."""
    rng = np.random.default_rng(8)
    L, H, d = 32, 1, 32
    qo = np.array([0, L])
    q = np.zeros((L, H, d))
    k = rng.standard_normal((L, H, d))
    v = rng.integers(-14, 15, (L, H, d)) * 2.0 ** -3
    do = rng.integers(-14, 15, (L, H, d)) * 2.0 ** -3
    v[0] = do[0] = 1.75   # block max 1.75 per column: scale 2^-8, every element exact
    out, lse = mx.mx_attention_fwd(q, k, v, qo, qo, 0.25, False)
    dq, dk, dv = mx.mx_attention_bwd(q, k, v, out, do, lse, qo, qo, 0.25, False)
    ref = oracle.attention_bwd(q, k, v, do, qo, qo, 0.25, "softmax", False)
    np.testing.assert_allclose(dv, ref[2], rtol=1e-13, atol=1e-13)
    assert np.all(dk == 0)


def _loop_mx_bwd(q, k, v, out, do, lse, qo, ko, scale, causal):
    """Independent per-element loop implementation for tiny inputs: scalar
    block scales from the bit-level definition and brute-force rounding."""
    def quant(vals):
        amax = max(abs(x) for x in vals)
        ex = -127 if amax == 0 else max(-127, min(127, math.frexp(amax)[1] - 1 - 8))
        return [_table_value(_nearest_code(x / 2.0 ** ex)) * 2.0 ** ex for x in vals]

    def quant_fit(vals):   # P and dS: the least exponent whose range holds the block (R8)
        amax = max(abs(x) for x in vals)
        ex = next(e for e in range(-127, 128) if amax <= 448.0 * 2.0 ** e)
        return [_table_value(_nearest_code(x / 2.0 ** ex)) * 2.0 ** ex for x in vals]
    T, H, d = q.shape
    Tk = k.shape[0]
    qr, kr, vr, dor = (np.zeros_like(x) for x in (q, k, v, do))
    for src, dst in ((q, qr), (k, kr), (v, vr), (do, dor)):
        for r in range(src.shape[0]):
            for h in range(H):
                for c0 in range(0, d, 32):
                    dst[r, h, c0:c0 + 32] = quant(list(src[r, h, c0:c0 + 32]))
    qc, doc, kc = np.zeros_like(q), np.zeros_like(do), np.zeros_like(k)
    for src, dst, off in ((q, qc, qo), (do, doc, qo), (k, kc, ko)):
        for b in range(len(off) - 1):
            for r0 in range(off[b], off[b + 1], 32):
                r1 = min(r0 + 32, off[b + 1])
                for h in range(H):
                    for col in range(d):
                        dst[r0:r1, h, col] = quant(list(src[r0:r1, h, col]))
    dq, dk, dv = np.zeros_like(q), np.zeros_like(k), np.zeros_like(v)
    for b in range(len(qo) - 1):
        lq, lk = qo[b + 1] - qo[b], ko[b + 1] - ko[b]
        for h in range(H):
            P = np.zeros((lq, lk))
            dS = np.zeros((lq, lk))
            for i in range(lq):
                dlt = sum(do[qo[b] + i, h, c] * out[qo[b] + i, h, c] for c in range(d))
                for j in range(lk):
                    if causal and j > i + lk - lq:
                        continue
                    s = scale * float(np.dot(qr[qo[b] + i, h], kr[ko[b] + j, h]))
                    P[i, j] = math.exp(s - lse[h, qo[b] + i])
                    dp = float(np.dot(dor[qo[b] + i, h], vr[ko[b] + j, h]))
                    dS[i, j] = P[i, j] * (dp - dlt)
            Pq, dSq, dSk = np.zeros_like(P), np.zeros_like(dS), np.zeros_like(dS)
            for j in range(lk):
                for r0 in range(0, lq, 32):
                    Pq[r0:r0 + 32, j] = quant_fit(list(P[r0:r0 + 32, j]))
                    dSq[r0:r0 + 32, j] = quant_fit(list(dS[r0:r0 + 32, j]))
            for i in range(lq):
                for c0 in range(0, lk, 32):
                    dSk[i, c0:c0 + 32] = quant_fit(list(dS[i, c0:c0 + 32]))
            for j in range(lk):
                for c in range(d):
                    dv[ko[b] + j, h, c] = sum(Pq[i, j] * doc[qo[b] + i, h, c] for i in range(lq))
                    dk[ko[b] + j, h, c] = scale * sum(dSq[i, j] * qc[qo[b] + i, h, c] for i in range(lq))
            for i in range(lq):
                for c in range(d):
                    dq[qo[b] + i, h, c] = scale * sum(dSk[i, j] * kc[ko[b] + j, h, c] for j in range(lk))
    return dq, dk, dv


@pytest.mark.parametrize("causal", [False, True])
def test_backward_matches_loop_implementation(causal):
    q, k, v, out, do, lse, qo, ko = _draw_bwd([2, 35], [36, 33], 1, 32, 21 + causal, causal)
    got = mx.mx_attention_bwd(q, k, v, out, do, lse, qo, ko, 0.3, causal)
    ref = _loop_mx_bwd(q, k, v, out, do, lse, qo, ko, 0.3, causal)
    for g, r in zip(got, ref):
        np.testing.assert_allclose(g, r, rtol=1e-9, atol=1e-11)


def test_mx_bwd_gates_separate_mistakes(monkeypatch):
    """The MXFP8 backward's GPU gates (tests.mx_util) are tight enough to see
    the plausible mistakes of a kernel: each, planted in the oracle, fails
    them by a factor of 2 or more -- relative L2 against the correct oracle,
    per tensor or per sequence, at least 2x the gate in some gradient, with
    the allowance for fp32 decisions (tests.mx_util.bwd_slack) taken off
    each element's difference as the GPU tests take it.
    Sequences start off the 32-row grid (where a block boundary counted from
    the packed row 0 differs from one counted from the sequence's start).

    Not among them: the axis or the block boundaries of P's and dS's own
    quantisation.  With the fitted exponent (R8) nothing saturates, so the
    partition only decides which elements below 2^-17 of a block's largest
    fall under E4M3's range, and those move the gradients by less than
    1e-5: the partition is not visible in the values (and does not matter
    to them)."""
    from tests.gpu_util import beyond_slack, rel_l2, seq_rel_l2
    from tests.mx_util import MX_GRAD_RTOL, MX_GRAD_SEQ_RTOL, bwd_slack
    lengths = [5, 37, 50, 71, 100, 130, 201]
    q, k, v, out, do, lse, qo, ko = _draw_bwd(lengths, lengths, 2, 128, 3, True)
    ref = mx.mx_attention_bwd(q, k, v, out, do, lse, qo, ko, 0.3, True)
    slack = bwd_slack(q, k, v, out, do, lse, qo, ko, 0.3, True)
    orig_keys, orig_mat = mx.mx_quantize_keys, mx.mx_quantize_matrix

    def mutant(name):
        calls = [0]

        def skip(which):   # mx_attention_bwd quantises P, dS (dK), dS (dQ) in turn
            def f(x, axis):
                calls[0] += 1
                return x if (calls[0] - 1) % 3 in which else orig_mat(x, axis)
            return f
        with monkeypatch.context() as m:
            if name == "blocks counted from packed row 0":
                m.setattr(mx, "mx_quantize_keys", lambda x, o: orig_keys(x, np.array([0, x.shape[0]])))
            elif name == "row images for the column operands":
                m.setattr(mx, "mx_quantize_keys", lambda x, o: mx.mx_quantize_rows(x))
                m.setattr(mx, "mx_dequantize_keys", mx.mx_dequantize_rows)
            elif name == "P not quantised":
                m.setattr(mx, "mx_quantize_matrix", skip((0,)))
            elif name == "dS not quantised for dK":
                m.setattr(mx, "mx_quantize_matrix", skip((1,)))
            elif name == "dS not quantised for dQ":
                m.setattr(mx, "mx_quantize_matrix", skip((2,)))
            return mx.mx_attention_bwd(q, k, v, out, do, lse, qo, ko, 0.3, True)

    for name in ("blocks counted from packed row 0", "row images for the column operands", "P not quantised",
                 "dS not quantised for dK", "dS not quantised for dQ"):
        got = [beyond_slack(g, r, a) for g, r, a in zip(mutant(name), ref, slack)]
        worst = max(max(rel_l2(g, r) / MX_GRAD_RTOL, seq_rel_l2(g, r, o)[0] / MX_GRAD_SEQ_RTOL)
                    for g, r, o in zip(got, ref, (qo, ko, ko)))
        assert worst >= 2.0, (name, worst)
