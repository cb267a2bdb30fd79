"""Pins for the oracle's mask/bias term (CPU only): additive fp32 bias and
the causal mask (key j hidden from query i when j > i + (Nk - Nq))."""
import math

import numpy as np
import pytest
import scipy.special

import fa06_inputs as fi
import oracle
from tests import bruteforce


def widen(bits):
    return fi.bf16_bits_to_f32(bits).astype(np.float64)


@pytest.mark.parametrize("Nq,Nk", [(6, 6), (4, 9), (9, 4), (1, 5)])
@pytest.mark.parametrize("with_bias", [False, True])
def test_bruteforce_causal_and_bias(Nq, Nk, with_bias):
    Q, K, V = fi.make_qkv(2, 2, Nq, Nk, 16, seed=60 + Nq + Nk, dv=8)
    rng = np.random.default_rng(61)
    bias = None
    if with_bias:
        # per-head bias broadcast over the batch, with a few -inf entries
        bias = rng.standard_normal((1, 2, Nq, Nk)).astype(np.float32)
        bias[0, 1, 0, -1] = -np.inf
    for causal in (False, True):
        O, L = oracle.attention_masked(Q, K, V, 0.3, causal=causal, bias=bias)
        Ob, Lb = bruteforce.attention(Q, K, V, 0.3, causal=causal, bias=bias)
        np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
        assert np.array_equal(np.isneginf(L), np.isneginf(Lb))
        fin = np.isfinite(Lb)
        np.testing.assert_allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)


def test_causal_row_is_attention_over_its_prefix():
    B, H, Nq, Nk, d = 1, 2, 12, 20, 128
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=62)
    sc = 1 / math.sqrt(d)
    O, L = oracle.attention_masked(Q, K, V, sc, causal=True)
    for i in range(Nq):
        n = i + (Nk - Nq) + 1
        Oi, Li = oracle.attention(np.ascontiguousarray(Q[:, :, i:i + 1]), np.ascontiguousarray(K[:, :, :n]),
                                  np.ascontiguousarray(V[:, :, :n]), sc)
        np.testing.assert_array_equal(O[:, :, i], Oi[:, :, 0])
        np.testing.assert_array_equal(L[:, :, i], Li[:, :, 0])


def test_rows_that_see_no_key():
    Q, K, V = fi.make_qkv(1, 1, 7, 3, 32, seed=63)
    O, L = oracle.attention_masked(Q, K, V, 0.2, causal=True)
    # rows 0..3 see nothing; row 4 sees key 0 only; row 6 sees all three
    assert np.all(O[0, 0, :4] == 0) and np.all(np.isneginf(L[0, 0, :4]))
    np.testing.assert_array_equal(O[0, 0, 4], widen(V)[0, 0, 0])
    Oa, La = oracle.attention(Q, K, V, 0.2)
    np.testing.assert_array_equal(O[0, 0, 6], Oa[0, 0, 6])
    bias = np.full((1, 1, 7, 3), -np.inf, np.float32)
    O2, L2 = oracle.attention_masked(Q, K, V, 0.2, bias=bias)
    assert np.all(O2 == 0) and np.all(np.isneginf(L2))


def test_constant_bias_shifts_lse_only():
    Q, K, V = fi.make_qkv(2, 3, 9, 31, 128, seed=64)
    sc = 1 / math.sqrt(128)
    rowc = np.random.default_rng(65).uniform(-5, 5, (2, 3, 9, 1)).astype(np.float32)
    O, L = oracle.attention(Q, K, V, sc)
    O2, L2 = oracle.attention_masked(Q, K, V, sc, bias=np.broadcast_to(rowc, (2, 3, 9, 31)))
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L2, L + rowc[..., 0].astype(np.float64), rtol=0, atol=1e-12)


def test_minus_inf_bias_removes_keys():
    Q, K, V = fi.make_qkv(1, 2, 10, 40, 128, seed=66)
    sc = 1 / math.sqrt(128)
    keep = np.random.default_rng(67).random(40) < 0.6
    bias = np.where(keep, 0.0, -np.inf).astype(np.float32)[None, None, None, :]
    O, L = oracle.attention_masked(Q, K, V, sc, bias=bias)
    Ok, Lk = oracle.attention(Q, np.ascontiguousarray(K[:, :, keep]), np.ascontiguousarray(V[:, :, keep]), sc)
    np.testing.assert_allclose(O, Ok, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lk, rtol=0, atol=1e-12)


def test_log_weight_bias_matches_library_softmax():
    Q, K, V = fi.make_qkv(1, 2, 16, 24, 64, seed=68)
    sc = float(np.float32(0.125))
    w = np.random.default_rng(69).uniform(0.1, 3.0, (1, 2, 16, 24))
    bias = np.log(w).astype(np.float32)
    O, L = oracle.attention_masked(Q, K, V, sc, bias=bias)
    S = np.float64(np.float32(sc)) * (widen(Q) @ np.swapaxes(widen(K), -1, -2)) + bias.astype(np.float64)
    np.testing.assert_allclose(O, scipy.special.softmax(S, axis=-1) @ widen(V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, scipy.special.logsumexp(S, axis=-1), rtol=0, atol=1e-12)


def test_broadcast_bias_equals_expanded_bias():
    Q, K, V = fi.make_qkv(2, 3, 5, 11, 32, seed=70)
    bias = np.random.default_rng(71).standard_normal((1, 3, 1, 11)).astype(np.float32)
    O1, L1 = oracle.attention_masked(Q, K, V, 0.2, causal=True, bias=bias)
    O2, L2 = oracle.attention_masked(Q, K, V, 0.2, causal=True,
                                     bias=np.ascontiguousarray(np.broadcast_to(bias, (2, 3, 5, 11))))
    assert np.array_equal(O1, O2) and np.array_equal(L1, L2)


def test_masked_rows_entry_matches_full():
    Q, K, V = fi.make_qkv(2, 2, 30, 50, 128, seed=72)
    bias = np.random.default_rng(73).standard_normal((2, 2, 30, 50)).astype(np.float32)
    O, L = oracle.attention_masked(Q, K, V, 0.1, causal=True, bias=bias)
    rows = np.array([0, 5, 29, 30, 77, 119], dtype=np.int64)
    Or, Lr = oracle.attention_masked(Q, K, V, 0.1, causal=True, bias=bias, rows=rows)
    assert np.array_equal(Or, O.reshape(-1, 128)[rows]) and np.array_equal(Lr, L.reshape(-1)[rows])
