"""Pins of the oracle's backward pass (CPU only).

The backward oracle is the chain rule of the score and output equations of
"FlashAttention'ı Anlamak Bölüm 1", section 0.2, written out row by row in
fp64.  It is pinned here to things outside its own code:

* central finite differences of an independent fp64 forward written in
  numpy (so every term of dQ, dK and dV, including the rank-one softmax term
  D, is checked against the derivative of the forward definition), with and
  without the causal mask and an additive bias, for a negative scale and for
  d_v != d;
* torch's float64 CPU autograd through scaled_dot_product_attention (a
  library routine);
* closed forms: one key (dQ = dK = 0, dV = sum of dO), zero scale (dQ = dK =
  0, dV = mean of dO over keys);
* invariants: sum_j dK_j = 0 (softmax is shift invariant in the keys),
  sum_j dV_j = sum_i dO_i (rows of P sum to one), exact doubling in dO, and
  D_i = dO_i . O_i with O from the forward oracle.
"""
import math

import numpy as np
import pytest

import fa06_inputs as fi
import oracle


def widen(bits):
    return fi.bf16_bits_to_f32(bits).astype(np.float64)


def forward64(Q, K, V, scale, causal=False, bias=None):
    """O = softmax(scale Q K^T + bias, causal bottom-right) V in float64 (numpy)."""
    S = scale * (Q @ np.swapaxes(K, -1, -2))
    if bias is not None:
        S = S + bias.astype(np.float64)
    Nq, Nk = S.shape[-2:]
    if causal:
        i = np.arange(Nq)[:, None]
        j = np.arange(Nk)[None, :]
        S = np.where(j > i + (Nk - Nq), -np.inf, S)
    m = S.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    E = np.exp(S - m)
    l = E.sum(axis=-1, keepdims=True)
    P = np.where(l > 0, E / np.where(l > 0, l, 1.0), 0.0)
    return P @ V


def finite_diff(Q, K, V, G, scale, causal, bias, eps=1e-5):
    """Central differences of L = sum(O * G) w.r.t. every element of Q, K, V."""
    grads = []
    args = [Q.copy(), K.copy(), V.copy()]
    for a in range(3):
        X = args[a]
        g = np.zeros_like(X)
        it = np.nditer(X, flags=["multi_index"])
        for _ in it:
            idx = it.multi_index
            old = X[idx]
            X[idx] = old + eps
            lp = float((forward64(*args, scale, causal, bias) * G).sum())
            X[idx] = old - eps
            lm = float((forward64(*args, scale, causal, bias) * G).sum())
            X[idx] = old
            g[idx] = (lp - lm) / (2 * eps)
        grads.append(g)
    return grads


FD_CASES = [
    # B, H, Nq, Nk, d, dv, scale, causal, with_bias, seed
    (1, 2, 5, 7, 16, 16, 0.3, False, False, 1),
    (2, 1, 6, 4, 8, 12, 0.5, False, False, 2),      # d_v != d, Nq > Nk
    (1, 2, 5, 9, 8, 8, 0.4, True, False, 3),       # causal, Nq < Nk
    (1, 1, 7, 4, 8, 8, 0.4, True, False, 4),       # causal, Nq > Nk: rows with no key
    (1, 2, 6, 6, 8, 8, -0.35, False, True, 5),     # negative scale, bias
    (1, 1, 5, 8, 8, 8, 0.3, True, True, 6),        # causal and bias
]


@pytest.mark.parametrize("B,H,Nq,Nk,d,dv,scale,causal,with_bias,seed", FD_CASES)
def test_gradients_match_finite_differences(B, H, Nq, Nk, d, dv, scale, causal, with_bias, seed):
    Q, K, _ = fi.make_qkv(B, H, Nq, Nk, d, seed=seed)
    V = fi.make_qkv(B, H, 1, Nk, dv, seed=seed + 100)[1]
    dO = fi.make_qkv(B, H, Nq, 1, dv, seed=seed + 200)[0]
    bias = None
    if with_bias:
        bias = np.random.default_rng(seed).standard_normal((B, H, Nq, Nk)).astype(np.float32)
    dQ, dK, dV, D, L = oracle.attention_bwd(Q, K, V, dO, scale, causal=causal, bias=bias)
    gQ, gK, gV = finite_diff(widen(Q), widen(K), widen(V), widen(dO), np.float64(np.float32(scale)), causal, bias)
    for name, a, b in (("dQ", dQ, gQ), ("dK", dK, gK), ("dV", dV, gV)):
        assert np.allclose(a, b, rtol=0, atol=2e-7), (name, float(np.abs(a - b).max()))


def test_matches_torch_autograd_float64():
    torch = pytest.importorskip("torch")
    B, H, Nq, Nk, d = 2, 3, 9, 11, 16
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=7)
    dO = fi.make_qkv(B, H, Nq, 1, d, seed=8)[0]
    bias = np.random.default_rng(9).standard_normal((1, H, Nq, Nk)).astype(np.float32)
    scale = float(np.float32(0.37))
    cases = [(False, None), (False, bias)]
    for causal, b in cases:
        q, k, v = (torch.tensor(widen(x), requires_grad=True) for x in (Q, K, V))
        mask = None if b is None else torch.tensor(b.astype(np.float64))
        o = torch.nn.functional.scaled_dot_product_attention(q, k, v, attn_mask=mask, scale=scale)
        o.backward(torch.tensor(widen(dO)))
        dQ, dK, dV, _, _ = oracle.attention_bwd(Q, K, V, dO, scale, causal=causal, bias=b)
        for a, t in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
            assert np.allclose(a, t.numpy(), rtol=0, atol=1e-12)
    # square causal: torch's is_causal (i >= j) equals the bottom-right diagonal when Nq = Nk
    Q, K, V = fi.make_qkv(1, 2, 10, 10, 16, seed=10)
    dO = fi.make_qkv(1, 2, 10, 1, 16, seed=11)[0]
    q, k, v = (torch.tensor(widen(x), requires_grad=True) for x in (Q, K, V))
    o = torch.nn.functional.scaled_dot_product_attention(q, k, v, is_causal=True, scale=scale)
    o.backward(torch.tensor(widen(dO)))
    dQ, dK, dV, _, _ = oracle.attention_bwd(Q, K, V, dO, scale, causal=True)
    for a, t in ((dQ, q.grad), (dK, k.grad), (dV, v.grad)):
        assert np.allclose(a, t.numpy(), rtol=0, atol=1e-12)


def test_single_key_closed_form():
    Q, K, V = fi.make_qkv(1, 2, 6, 1, 16, seed=12)
    dO = fi.make_qkv(1, 2, 6, 1, 16, seed=13)[0]
    dQ, dK, dV, D, _ = oracle.attention_bwd(Q, K, V, dO, 0.3)
    assert np.all(dQ == 0) and np.all(dK == 0)
    assert np.allclose(dV[:, :, 0], widen(dO).sum(axis=2), rtol=0, atol=1e-12)


def test_zero_scale_closed_form():
    Nk = 8
    Q, K, V = fi.make_qkv(1, 2, 5, Nk, 16, seed=14)
    dO = fi.make_qkv(1, 2, 5, 1, 16, seed=15)[0]
    dQ, dK, dV, _, _ = oracle.attention_bwd(Q, K, V, dO, 0.0)
    assert np.all(dQ == 0) and np.all(dK == 0)
    want = np.repeat(widen(dO).sum(axis=2, keepdims=True) / Nk, Nk, axis=2)
    assert np.allclose(dV, want, rtol=0, atol=1e-12)


@pytest.mark.parametrize("causal", [False, True])
def test_invariants(causal):
    B, H, Nq, Nk, d = 2, 2, 12, 10, 16
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=16)
    dO = fi.make_qkv(B, H, Nq, 1, d, seed=17)[0]
    dQ, dK, dV, D, L = oracle.attention_bwd(Q, K, V, dO, 0.25, causal=causal)
    # softmax is unchanged when one vector is added to every key: sum_j dK_j = 0
    assert np.allclose(dK.sum(axis=2), 0.0, rtol=0, atol=1e-12)
    # rows of P sum to one: sum_j dV_j = sum over the rows that see a key of dO_i
    sees = np.isfinite(L)
    G = widen(dO) * sees[..., None]
    assert np.allclose(dV.sum(axis=2), G.sum(axis=2), rtol=0, atol=1e-12)
    # D_i = dO_i . O_i with O from the forward oracle
    O, Lf = oracle.attention_masked(Q, K, V, 0.25, causal=causal)
    assert np.allclose(D, (widen(dO) * O).sum(axis=-1), rtol=0, atol=1e-12)
    assert np.array_equal(np.isneginf(L), np.isneginf(Lf))
    assert np.allclose(L[sees], Lf[sees], rtol=0, atol=0)
    # exact doubling: 2*dO is exact in bf16, and every gradient doubles exactly
    dO2 = fi.f32_to_bf16_bits(2 * fi.bf16_bits_to_f32(dO))
    g2 = oracle.attention_bwd(Q, K, V, dO2, 0.25, causal=causal)
    for a, b in zip(g2[:3], (dQ, dK, dV)):
        assert np.array_equal(a, 2 * b)


@pytest.mark.parametrize("bias_kind", [None, "full", "per_key"])
def test_sampled_entry_points_equal_the_full_backward(bias_kind):
    B, H, Nq, Nk, d = 2, 3, 40, 50, 16
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=18)
    dO = fi.make_qkv(B, H, Nq, 1, d, seed=19)[0]
    rng = np.random.default_rng(22)
    bias = None
    if bias_kind == "full":
        bias = rng.standard_normal((B, H, Nq, Nk)).astype(np.float32)
        bias[1, 2, :, 30:] = -np.inf
        bias[0, 1, 5, :] = -np.inf          # a row that sees no key
    elif bias_kind == "per_key":
        bias = (3 * rng.standard_normal((1, H, 1, Nk))).astype(np.float32)
    for causal in (False, True):
        dQ, dK, dV, _, _ = oracle.attention_bwd(Q, K, V, dO, 0.2, causal=causal, bias=bias)
        rows = np.array([0, 7, 39, 40, 45, 119, 239], dtype=np.int64)
        assert np.array_equal(oracle.attention_bwd_dq_rows(Q, K, V, dO, 0.2, rows, causal=causal, bias=bias),
                              dQ.reshape(-1, d)[rows])
        keys = np.array([0, 49, 50, 77, 299, 77], dtype=np.int64)
        k1, v1 = oracle.attention_bwd_dkdv_keys(Q, K, V, dO, 0.2, keys, causal=causal, bias=bias)
        assert np.allclose(k1, dK.reshape(-1, d)[keys], rtol=0, atol=1e-13)
        assert np.allclose(v1, dV.reshape(-1, d)[keys], rtol=0, atol=1e-13)
        if bias_kind == "full":
            assert np.all(dQ[0, 1, 5] == 0)


def test_bad_arguments():
    Q, K, V = fi.make_qkv(1, 1, 4, 4, 8, seed=20)
    dO = fi.make_qkv(1, 1, 4, 1, 8, seed=21)[0]
    with pytest.raises(TypeError):
        oracle.attention_bwd(Q, K, V, dO[..., :4], 0.3)
    with pytest.raises(ValueError):
        oracle.attention_bwd_dq_rows(Q, K, V, dO, 0.3, np.array([4]))
    with pytest.raises(ValueError):
        oracle.attention_bwd_dkdv_keys(Q, K, V, dO, 0.3, np.array([-1]))
