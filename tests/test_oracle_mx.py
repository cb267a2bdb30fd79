"""Pins of the oracle's MXFP8 encoding (CPU only).

Values follow from the E4M3 / E8M0 format definitions of the OCP
microscaling specification (bias 7, 3 mantissa bits, subnormals below 2^-6,
NaN at S.1111.111, no infinity; E8M0 = 2^(s-127)), checked independently of
the table the oracle builds: by the bit-field formula written here, by
exhaustive round trips, by brute-force nearest search, and by the error
bound of round-to-nearest.
"""
import math

import numpy as np
import pytest

from oracle import mx


def formula(code):
    s = -1.0 if code & 0x80 else 1.0
    e, m = (code >> 3) & 15, code & 7
    return s * (m / 8 * 2 ** -6 if e == 0 else (1 + m / 8) * 2.0 ** (e - 7))


def test_known_codes():
    assert mx.e4m3_decode(np.array([0x38]))[0] == 1.0
    assert mx.e4m3_decode(np.array([0x7E]))[0] == 448.0
    assert mx.e4m3_decode(np.array([0x01]))[0] == 2.0 ** -9
    assert mx.e4m3_decode(np.array([0x08]))[0] == 2.0 ** -6
    assert mx.e4m3_decode(np.array([0x77]))[0] == 240.0
    assert mx.e4m3_decode(np.array([0xC2]))[0] == -2.5
    assert np.isnan(mx.e4m3_decode(np.array([0x7F, 0xFF]))).all()
    for code in range(256):
        if code & 0x7F == 0x7F:
            continue
        assert mx.e4m3_decode(np.array([code]))[0] == formula(code)


def test_every_finite_code_round_trips():
    codes = np.array([c for c in range(256) if c & 0x7F != 0x7F], dtype=np.uint8)
    assert np.array_equal(mx.e4m3_encode(mx.e4m3_decode(codes)), codes)


def test_encode_is_nearest_with_ties_to_even_and_saturates():
    finite = np.array([formula(c) for c in range(0x7F)])  # non-negative codes 0..126
    rng = np.random.default_rng(0)
    xs = np.concatenate([rng.uniform(0, 460, 3000), rng.uniform(0, 2 ** -5, 1000),
                         (finite[1:] + finite[:-1]) / 2])          # every midpoint: a tie
    got = mx.e4m3_encode(xs)
    for x, c in zip(xs, got):
        d = np.abs(finite - min(x, 448.0))
        best = np.flatnonzero(d == d.min())
        want = best[0] if len(best) == 1 else [b for b in best if b % 2 == 0][0]
        assert c == want, (x, c, want)
    assert mx.e4m3_encode(np.array([500.0, -1e9, -0.0]))[0] == 0x7E
    assert mx.e4m3_encode(np.array([-1e9]))[0] == 0xFE
    assert mx.e4m3_encode(np.array([-0.0]))[0] == 0x80


def test_block_scale_choice_and_error_bound():
    rng = np.random.default_rng(1)
    x = rng.standard_normal((5, 7, 64)) * np.exp2(rng.integers(-20, 20, (5, 7, 1)))
    q, s = mx.mx_quantize(x)
    assert q.shape == x.shape and s.shape == (5, 7, 2)
    amax = np.abs(x.reshape(5, 7, 2, 32)).max(-1)
    assert np.array_equal(s.astype(int) - 127, np.floor(np.log2(amax)).astype(int) - 8)
    d = mx.mx_dequantize(q, s)
    X = np.repeat(mx.e8m0_decode(s), 32, axis=-1)
    # round to nearest: error at most half a unit of the E4M3 grid at that
    # magnitude (relative 2^-4 for normals, 2^-10 * X for subnormals), except
    # saturated values, which land on 448 * X
    bound = np.maximum(np.abs(x) * 2.0 ** -4, X * 2.0 ** -10)
    sat = np.abs(x) / X > 448
    assert np.all(np.abs(d - x)[~sat] <= bound[~sat] * (1 + 1e-12))
    assert np.all(np.abs(d[sat]) == 448 * X[sat])


def test_zero_block_and_idempotence():
    x = np.zeros((2, 32))
    x[1, 3] = 3.0
    q, s = mx.mx_quantize(x)
    assert s[0, 0] == 0 and np.all(q[0] == 0)
    assert s[1, 0] == 127 + 1 - 8
    rng = np.random.default_rng(2)
    y = rng.standard_normal((4, 96)) * 3
    q, s = mx.mx_quantize(y)
    q2, s2 = mx.mx_quantize(mx.mx_dequantize(q, s))
    assert np.array_equal(q, q2) and np.array_equal(s, s2)


def test_attention_inputs_layout_and_exact_bf16():
    rng = np.random.default_rng(3)
    Q = rng.standard_normal((1, 2, 5, 64))
    K = rng.standard_normal((1, 2, 9, 64))
    V = rng.standard_normal((1, 2, 9, 64))
    (q8, qs, k8, ks, vt8, vs), (Qb, Kb, Vb) = mx.quantize_attention_inputs(Q, K, V, ldv=64)
    assert vt8.shape == (1, 2, 64, 64) and vs.shape == (1, 2, 64, 2)
    assert np.all(vt8[..., 9:] == 0)                # padded keys are zero
    # V's blocks run along the keys: dequantizing the transposed encoding
    # and transposing back gives the V the attention oracle sees
    Vd = np.swapaxes(mx.mx_dequantize(vt8, vs), -1, -2)[:, :, :9]
    widen = lambda b: (b.astype(np.uint32) << 16).view(np.float32).astype(np.float64)
    assert np.array_equal(widen(Vb), Vd)
    assert np.array_equal(widen(Qb), mx.mx_dequantize(q8, qs))
    assert np.array_equal(widen(Kb), mx.mx_dequantize(k8, ks))
    with pytest.raises(ValueError):
        mx.as_bf16_bits(np.array([1.0 + 2.0 ** -10]))
