"""Pins for the fp64 CPU oracle (CPU only).

The oracle is checked against things other than itself: a brute-force
evaluation on tiny inputs, library softmax/logsumexp routines, closed forms
(identical keys, constant value columns, one key, zero scale, two keys),
invariances of softmax (shift, permutation), the hardmax limit, the
online-softmax recurrence printed in the 5090 article's "v1" section, and
the Gaussian statistics of the synthetic workloads.  Each is chosen so that a
dropped term, a wrong sign, a wrong index or stride, or a transposed operand
in the oracle fails at least one of them.
"""
import math

import numpy as np
import pytest
import scipy.special

import fa06_inputs as fi
import oracle
from tests import bruteforce

pytestmark = pytest.mark.filterwarnings("ignore::RuntimeWarning")


def widen(bits):
    return fi.bf16_bits_to_f32(bits).astype(np.float64)


def bits_of(x):
    """bf16 bits of values that are exactly representable in bf16."""
    b = fi.f32_to_bf16_bits(np.asarray(x, dtype=np.float32))
    assert np.array_equal(widen(b), np.asarray(x, dtype=np.float64)), "value not exact in bf16"
    return b


def scale_of(d):
    return float(np.float32(1.0 / math.sqrt(d)))


@pytest.mark.parametrize("B,H,Nq,Nk,d,dv,scale,seed", [
    (1, 1, 3, 5, 128, 128, None, 1),
    (2, 3, 5, 7, 16, 8, None, 2),      # multi-head, dv != d, Nk != d
    (1, 2, 4, 16, 128, 128, None, 3),
    (1, 1, 6, 9, 32, 48, -0.25, 4),    # negative scale, dv > d
    (2, 1, 2, 1, 8, 8, None, 5),       # one key
])
def test_bruteforce_tiny(B, H, Nq, Nk, d, dv, scale, seed):
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=seed, dv=dv)
    sc = scale_of(d) if scale is None else scale
    O, L = oracle.attention(Q, K, V, sc)
    Ob, Lb = bruteforce.attention(Q, K, V, sc)
    np.testing.assert_allclose(O, Ob, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, Lb, rtol=0, atol=1e-12)


def test_library_softmax_logsumexp():
    Q, K, V = fi.make_qkv(2, 2, 64, 96, 128, seed=11)
    sc = scale_of(128)
    O, L = oracle.attention(Q, K, V, sc)
    S = np.float32(sc).astype(np.float64) * (widen(Q) @ np.swapaxes(widen(K), -1, -2))
    P = scipy.special.softmax(S, axis=-1)
    np.testing.assert_allclose(O, P @ widen(V), rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, scipy.special.logsumexp(S, axis=-1), rtol=0, atol=1e-12)


def test_rows_of_p_sum_to_one():
    # With V the Nk x Nk identity, O = P V = P: the oracle's probabilities.
    B, H, Nq, Nk, d = 1, 2, 8, 24, 128
    Q, K, _ = fi.make_qkv(B, H, Nq, Nk, d, seed=12)
    V = np.broadcast_to(bits_of(np.eye(Nk)), (B, H, Nk, Nk)).copy()
    P, _ = oracle.attention(Q, K, V, scale_of(d))
    assert np.all(P > 0)
    np.testing.assert_allclose(P.sum(-1), 1.0, rtol=0, atol=1e-12)
    S = np.float32(scale_of(d)).astype(np.float64) * (widen(Q) @ np.swapaxes(widen(K), -1, -2))
    E = np.exp(S - S.max(-1, keepdims=True))
    np.testing.assert_allclose(P, E / E.sum(-1, keepdims=True), rtol=0, atol=1e-12)


def test_identical_keys_give_mean_of_v():
    B, H, Nq, Nk, d = 1, 2, 6, 40, 128
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=13)
    K[:] = K[:, :, :1, :]
    sc = scale_of(d)
    O, L = oracle.attention(Q, K, V, sc)
    np.testing.assert_allclose(O, np.broadcast_to(widen(V).mean(axis=2, keepdims=True), O.shape),
                               rtol=0, atol=1e-12)
    qk = np.einsum("bhid,bhd->bhi", widen(Q), widen(K)[:, :, 0, :])
    np.testing.assert_allclose(L, np.float64(np.float32(sc)) * qk + math.log(Nk), rtol=0, atol=1e-12)


def test_constant_v_column():
    B, H, Nq, Nk, d = 2, 1, 7, 33, 128
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=14)
    gam = [1.5, -3.0, 0.0078125, 96.0]
    for c, g in enumerate(gam):
        V[..., 5 * c] = bits_of(g)
    O, _ = oracle.attention(Q, K, V, scale_of(d))
    for c, g in enumerate(gam):
        np.testing.assert_allclose(O[..., 5 * c], g, rtol=1e-12, atol=0)


def test_one_key():
    Q, K, V = fi.make_qkv(2, 2, 5, 1, 128, seed=15)
    sc = scale_of(128)
    O, L = oracle.attention(Q, K, V, sc)
    assert np.array_equal(O, np.broadcast_to(widen(V), O.shape))
    dots = np.array([[[math.fsum(a * b for a, b in zip(widen(Q)[b, h, i], widen(K)[b, h, 0]))
                       for i in range(5)] for h in range(2)] for b in range(2)])
    np.testing.assert_allclose(L, np.float64(np.float32(sc)) * dots, rtol=1e-15, atol=1e-15)


def test_two_keys_closed_form():
    # softmax over two logits: O = v0 + (v1 - v0) * sigmoid(s1 - s0), LSE = logaddexp(s0, s1)
    Q, K, V = fi.make_qkv(1, 1, 9, 2, 64, seed=16)
    sc = scale_of(64)
    O, L = oracle.attention(Q, K, V, sc)
    q, k, v = widen(Q)[0, 0], widen(K)[0, 0], widen(V)[0, 0]
    s = np.float64(np.float32(sc)) * (q @ k.T)
    g = scipy.special.expit(s[:, 1] - s[:, 0])[:, None]
    np.testing.assert_allclose(O[0, 0], v[0] + (v[1] - v[0]) * g, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L[0, 0], np.logaddexp(s[:, 0], s[:, 1]), rtol=0, atol=1e-12)


def test_zero_scale_is_uniform():
    Q, K, V = fi.make_qkv(1, 3, 4, 50, 128, seed=17)
    O, L = oracle.attention(Q, K, V, 0.0)
    np.testing.assert_allclose(O, np.broadcast_to(widen(V).mean(axis=2, keepdims=True), O.shape),
                               rtol=0, atol=1e-12)
    np.testing.assert_allclose(L, math.log(50), rtol=0, atol=1e-12)


def test_shift_invariance():
    # Integer-valued inputs keep K + u exact in bf16.
    rng = np.random.default_rng(18)
    B, H, Nq, Nk, d = 1, 2, 5, 30, 128
    Qf = rng.integers(-3, 4, size=(B, H, Nq, d)).astype(np.float32) / 8
    Kf = rng.integers(-8, 9, size=(B, H, Nk, d)).astype(np.float32) / 8
    u = rng.integers(-4, 5, size=(B, H, 1, d)).astype(np.float32) / 8
    Vb = fi.make_qkv(B, H, 1, Nk, d, seed=19)[2]
    sc = scale_of(d)
    O1, L1 = oracle.attention(bits_of(Qf), bits_of(Kf), Vb, sc)
    O2, L2 = oracle.attention(bits_of(Qf), bits_of(Kf + u), Vb, sc)
    np.testing.assert_allclose(O2, O1, rtol=0, atol=1e-10)
    qu = np.einsum("bhid,bhd->bhi", Qf.astype(np.float64), u[:, :, 0, :].astype(np.float64))
    np.testing.assert_allclose(L2, L1 + np.float64(np.float32(sc)) * qu, rtol=0, atol=1e-10)


def test_permutation_invariance():
    B, H, Nq, Nk, d = 1, 2, 11, 37, 128
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=20)
    sc = scale_of(d)
    O, L = oracle.attention(Q, K, V, sc)
    rng = np.random.default_rng(21)
    pk = rng.permutation(Nk)
    O2, L2 = oracle.attention(Q, K[:, :, pk], V[:, :, pk], sc)
    np.testing.assert_allclose(O2, O, rtol=0, atol=1e-12)
    np.testing.assert_allclose(L2, L, rtol=0, atol=1e-12)
    pq = rng.permutation(Nq)
    O3, L3 = oracle.attention(np.ascontiguousarray(Q[:, :, pq]), K, V, sc)
    assert np.array_equal(O3, O[:, :, pq]) and np.array_equal(L3, L[:, :, pq])
    # swapping heads swaps the outputs (catches a wrong per-head stride)
    O4, L4 = oracle.attention(np.ascontiguousarray(Q[:, ::-1]), np.ascontiguousarray(K[:, ::-1]),
                              np.ascontiguousarray(V[:, ::-1]), sc)
    assert np.array_equal(O4, O[:, ::-1]) and np.array_equal(L4, L[:, ::-1])


def test_hardmax_limit():
    B, H, Nq, Nk, d = 1, 1, 32, 64, 128
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=22)
    big = 1000.0
    O, L = oracle.attention(Q, K, V, big)
    assert np.all(np.isfinite(O)) and np.all(np.isfinite(L))
    dots = widen(Q)[0, 0] @ widen(K)[0, 0].T
    srt = np.sort(dots, axis=1)
    gap = srt[:, -1] - srt[:, -2]
    am = dots.argmax(axis=1)
    ok = gap > 0.05            # exp(-50) is far below the tolerance
    assert ok.sum() >= 16
    np.testing.assert_allclose(O[0, 0][ok], widen(V)[0, 0][am[ok]], rtol=0, atol=1e-6)
    np.testing.assert_allclose(L[0, 0][ok], big * srt[ok, -1], rtol=1e-12, atol=0)


def _online(q, k, v, sigma, splits, normalise_each_step):
    """The recurrence of the 5090 article ("v1", online softmax) on one row.

    Running max m, running denominator (called l here) and output, updated
    block by block; either renormalised at every step (the printed form) or
    only at the end (the deferred form of the B200 article's partition
    section).
    """
    m, l, o = -math.inf, 0.0, np.zeros(v.shape[1])
    for a, b in zip(splits[:-1], splits[1:]):
        s = sigma * (k[a:b] @ q)
        m_new = max(m, s.max())
        e = np.exp(s - m_new)
        l_new = l * math.exp(m - m_new) + e.sum()
        if normalise_each_step:
            o = o * (l / l_new) * math.exp(m - m_new) + (e / l_new) @ v[a:b]
        else:
            o = o * math.exp(m - m_new) + e @ v[a:b]
        m, l = m_new, l_new
    if not normalise_each_step:
        o = o / l
    return o, m + math.log(l)


@pytest.mark.parametrize("normalise_each_step", [True, False])
def test_two_pass_equals_online_recurrence(normalise_each_step):
    B, H, Nq, Nk, d = 1, 1, 6, 57, 128
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=23, k_scale=3.0, offset_frac=0.1, offset=2.0)
    sc = scale_of(d)
    O, L = oracle.attention(Q, K, V, sc)
    q, k, v = widen(Q)[0, 0], widen(K)[0, 0], widen(V)[0, 0]
    rng = np.random.default_rng(24)
    for i in range(Nq):
        for _ in range(3):
            cuts = sorted(rng.choice(np.arange(1, Nk), size=rng.integers(1, 8), replace=False))
            splits = [0, *cuts, Nk]
            o, lse = _online(q[i], k, v, np.float64(np.float32(sc)), splits, normalise_each_step)
            np.testing.assert_allclose(o, O[0, 0, i], rtol=0, atol=1e-12)
            assert abs(lse - L[0, 0, i]) < 1e-12


def test_rows_entry_matches_full():
    Q, K, V = fi.make_qkv(2, 3, 40, 70, 128, seed=25)
    sc = scale_of(128)
    O, L = oracle.attention(Q, K, V, sc)
    rows = np.array([0, 1, 39, 40, 117, 239], dtype=np.int64)
    Or, Lr = oracle.attention_rows(Q, K, V, sc, rows)
    assert np.array_equal(Or, O.reshape(-1, 128)[rows]) and np.array_equal(Lr, L.reshape(-1)[rows])


def test_bad_arguments_rejected():
    Q, K, V = fi.make_qkv(1, 1, 4, 4, 16, seed=26)
    with pytest.raises(ValueError):
        oracle.attention(Q, K[:, :, :0], V[:, :, :0], 0.25)          # Nk = 0
    with pytest.raises(ValueError):
        oracle.attention_rows(Q, K, V, 0.25, np.array([4], dtype=np.int64))  # row out of range


def test_gaussian_statistics_tiny_workload():
    # For iid N(0,1) q, k and scale 1/sqrt(d), a logit has variance |q|^2/d,
    # so E[LSE] ~= ln Nk + 1/2 and std(O) ~= sqrt(e / Nk).
    w = fi.WORKLOADS["tiny_256"]
    Q, K, V = fi.make_workload(w)
    O, L = oracle.attention(Q, K, V, w.scale)
    assert abs(L.mean() - (math.log(w.Nk) + 0.5)) < 0.02
    assert abs(O.std() / math.sqrt(math.e / w.Nk) - 1.0) < 0.1


def test_gaussian_statistics_rtx5090_shape_sampled():
    w = fi.WORKLOADS["rtx5090_q4096_kv8192"]
    Q, K, V = fi.make_workload(w)
    rows = fi.sample_rows(w.B, w.H, w.Nq, 128, seed=w.seed)
    O, L = oracle.attention_rows(Q, K, V, w.scale, rows)
    assert abs(L.mean() - (math.log(w.Nk) + 0.5)) < 0.02
    assert abs(O.std() / math.sqrt(math.e / w.Nk) - 1.0) < 0.1
