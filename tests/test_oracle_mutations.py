"""The oracle's pins catch plausible mistakes (CPU only).

Each case plants one mistake in a copy of the oracle's C source (a dropped
term, a wrong sign, a transposed operand, a wrong index or stride), builds the
mutant in a temporary directory and checks that at least one pin -- brute
force, closed form, library routine or a limit -- rejects it.  Every mutant
keeps all memory accesses inside the input buffers for the shapes used here.
"""
import ctypes
import math
import os
import subprocess

import numpy as np
import pytest
import scipy.special

import fa06_inputs as fi
import oracle
from tests import bruteforce

SRC = os.path.join(os.path.dirname(oracle.__file__), "fa_oracle.c")

MUTATIONS = {
    "scale dropped": ("s[j] = sigma * dot;", "s[j] = dot;"),
    "exp sign flipped": ("s[j] = exp(s[j] - m);", "s[j] = exp(s[j] + m);"),
    "K transposed": ("widen_bf16(K[j * d + c]);\n        s[j] = sigma * dot;",
                     "widen_bf16(K[c * n_vis + j]);\n        s[j] = sigma * dot;"),
    "LSE max term dropped": ("    *lse = m + log(l);\n}", "    *lse = log(l);\n}"),
    "no normalisation": ("for (int64_t c = 0; c < dv; ++c) o[c] /= l;", ""),
    "always head 0": ("const int64_t bh = flat / Nq;", "const int64_t bh = 0;"),
    "Q ignores head": ("attend_one_row(Q + flat * d,", "attend_one_row(Q + (flat % Nq) * d,"),
    "min instead of max": ("if (s[j] > m) m = s[j];", "if (s[j] < m) m = s[j];"),
    "count instead of sum": ("        l += s[j];", "        l += 1.0;"),
    "V row stride off by one": ("o[c] += s[j] * widen_bf16(V[j * dv + c]);",
                                "o[c] += s[j] * widen_bf16(V[(j > 0 ? j - 1 : 0) * dv + c]);"),
}

# Mistakes in the mask/bias term, caught by the masked pins.
MASK_MUTATIONS = {
    "causal diagonal off by one": ("n_vis = i + (Nk - Nq) + 1;", "n_vis = i + (Nk - Nq);"),
    "causal diagonal not aligned to the last key": ("n_vis = i + (Nk - Nq) + 1;", "n_vis = i + 1;"),
    "bias subtracted": ("if (bias_row) s[j] += (double)bias_row[j];", "if (bias_row) s[j] -= (double)bias_row[j];"),
    "bias head stride ignored": ("(bh % H) * sh", "0 * sh"),
}


# Mistakes in the backward pass, caught by finite differences of an
# independent forward (tests/test_oracle_bwd.py).
BWD_MUTATIONS = {
    "softmax Jacobian term D dropped": (
        "const double ds = p[j] * (dp[j] - Di);\n                    for (int64_t c = 0; c < d; ++c) {\n"
        "                        dQi[c]",
        "const double ds = p[j] * dp[j];\n                    for (int64_t c = 0; c < d; ++c) {\n"
        "                        dQi[c]"),
    "dK without the scale": ("dKh[j * d + c] += sigma * ds * widen_bf16(qi[c]);",
                             "dKh[j * d + c] += ds * widen_bf16(qi[c]);"),
    "dK from K instead of Q": ("dKh[j * d + c] += sigma * ds * widen_bf16(qi[c]);",
                               "dKh[j * d + c] += sigma * ds * widen_bf16(Kh[j * d + c]);"),
    "dV weighted by dP instead of P": ("dVh[j * dv + c] += p[j] * widen_bf16(dOi[c]);",
                                       "dVh[j * dv + c] += dp[j] * widen_bf16(dOi[c]);"),
    "D not weighted by P": ("Di += p[j] * dot;", "Di += dot;"),
    "probabilities not normalised": ("for (int64_t j = 0; j < n_vis; ++j) p[j] /= l;", ""),
    "backward scores from a transposed K": ("widen_bf16(K[j * d + c]);\n        p[j] = sigma * dot;",
                                            "widen_bf16(K[c * n_vis + j]);\n        p[j] = sigma * dot;"),
    "dP ignores the value row": ("dot += widen_bf16(dOi[c]) * widen_bf16(V[j * dv + c]);",
                                 "dot += widen_bf16(dOi[c]) * widen_bf16(V[c]);"),
}


def build_mutant(tmp_path, name, old, new):
    src = open(SRC).read()
    assert src.count(old) == 1, f"mutation anchor for {name!r} not unique"
    path = tmp_path / "mutant.c"
    path.write_text(src.replace(old, new))
    lib = tmp_path / "libmutant.so"
    subprocess.run(["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared", "-ffp-contract=off",
                    str(path), "-o", str(lib), "-lm"], check=True)
    so = ctypes.CDLL(str(lib))
    i64, p = ctypes.c_int64, ctypes.c_void_p
    so.oracle_attn_fp64.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_float, p, p]
    so.oracle_attn_fp64.restype = ctypes.c_int
    so.oracle_attn_masked_fp64.argtypes = [p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                           ctypes.c_int, p, i64, i64, i64, p, i64, p, p]
    so.oracle_attn_masked_fp64.restype = ctypes.c_int
    so.oracle_attn_bwd_fp64.argtypes = [p, p, p, p, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                        ctypes.c_int, p, i64, i64, i64, p, p, p, p, p]
    so.oracle_attn_bwd_fp64.restype = ctypes.c_int

    def attention(Q, K, V, scale):
        B, H, Nq, d = Q.shape
        Nk, dv = K.shape[2], V.shape[3]
        Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
        O = np.empty((B, H, Nq, dv))
        L = np.empty((B, H, Nq))
        rc = so.oracle_attn_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data, B, H, Nq, Nk, d, dv,
                                 ctypes.c_float(scale), O.ctypes.data, L.ctypes.data)
        assert rc == 0
        return O, L

    def masked(Q, K, V, scale, causal, bias):
        B, H, Nq, d = Q.shape
        Nk, dv = K.shape[2], V.shape[3]
        full = np.ascontiguousarray(np.broadcast_to(bias, (B, H, Nq, Nk)).astype(np.float32))
        O = np.empty((B, H, Nq, dv))
        L = np.empty((B, H, Nq))
        rc = so.oracle_attn_masked_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data, B, H, Nq, Nk, d, dv,
                                        ctypes.c_float(scale), int(causal), full.ctypes.data,
                                        H * Nq * Nk, Nq * Nk, Nk, None, B * H * Nq, O.ctypes.data, L.ctypes.data)
        assert rc == 0
        return O, L
    def bwd(Q, K, V, dO, scale, causal=False):
        B, H, Nq, d = Q.shape
        Nk, dv = K.shape[2], V.shape[3]
        out = [np.empty((B, H, Nq, d)), np.empty((B, H, Nk, d)), np.empty((B, H, Nk, dv)),
               np.empty((B, H, Nq)), np.empty((B, H, Nq))]
        rc = so.oracle_attn_bwd_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data, dO.ctypes.data,
                                     B, H, Nq, Nk, d, dv, ctypes.c_float(scale), int(causal), None, 0, 0, 0,
                                     *(a.ctypes.data for a in out))
        assert rc == 0
        return out
    attention.masked = masked
    attention.bwd = bwd
    return attention


def widen(bits):
    return fi.bf16_bits_to_f32(bits).astype(np.float64)


def pins_pass(attention):
    """True when every pin accepts the implementation."""
    ok = True
    # brute force, several heads and batches, Nk != d
    Q, K, V = fi.make_qkv(2, 3, 5, 7, 16, seed=2)
    O, L = attention(Q, K, V, 0.25)
    Ob, Lb = bruteforce.attention(Q, K, V, 0.25)
    ok &= np.allclose(O, Ob, rtol=0, atol=1e-12) and np.allclose(L, Lb, rtol=0, atol=1e-12)
    # library softmax / logsumexp on a larger head
    Q, K, V = fi.make_qkv(1, 2, 24, 40, 32, seed=3)
    sc = float(np.float32(1 / math.sqrt(32)))
    O, L = attention(Q, K, V, sc)
    S = np.float64(np.float32(sc)) * (widen(Q) @ np.swapaxes(widen(K), -1, -2))
    ok &= np.allclose(O, scipy.special.softmax(S, axis=-1) @ widen(V), rtol=0, atol=1e-12)
    ok &= np.allclose(L, scipy.special.logsumexp(S, axis=-1), rtol=0, atol=1e-12)
    # hardmax limit: large logits must neither overflow nor mix
    Q, K, V = fi.make_qkv(1, 1, 16, 32, 64, seed=4)
    with np.errstate(all="ignore"):
        O, L = attention(Q, K, V, 500.0)
    dots = widen(Q)[0, 0] @ widen(K)[0, 0].T
    srt = np.sort(dots, axis=1)
    sel = (srt[:, -1] - srt[:, -2]) > 0.1
    am = dots.argmax(axis=1)
    ok &= bool(np.all(np.isfinite(O))) and np.allclose(O[0, 0][sel], widen(V)[0, 0][am[sel]], atol=1e-6)
    return bool(ok)


def test_unmutated_oracle_passes_the_pins():
    assert pins_pass(oracle.attention)


@pytest.mark.parametrize("name", list(MUTATIONS))
def test_mutant_is_caught(tmp_path, name):
    old, new = MUTATIONS[name]
    attention = build_mutant(tmp_path, name, old, new)
    assert not pins_pass(attention), f"mutation {name!r} was not detected by any pin"


def masked_pins_pass(masked):
    """Brute force with a causal mask (Nq < Nk and Nq > Nk) and a per-head bias."""
    ok = True
    rng = np.random.default_rng(5)
    for Nq, Nk in ((4, 9), (9, 4)):
        Q, K, V = fi.make_qkv(1, 2, Nq, Nk, 16, seed=6)
        bias = rng.standard_normal((1, 2, Nq, Nk)).astype(np.float32)
        O, L = masked(Q, K, V, 0.3, True, bias)
        Ob, Lb = bruteforce.attention(Q, K, V, 0.3, causal=True, bias=bias)
        fin = np.isfinite(Lb)
        ok &= np.allclose(O, Ob, rtol=0, atol=1e-12) and np.array_equal(np.isfinite(L), fin)
        ok &= np.allclose(L[fin], Lb[fin], rtol=0, atol=1e-12)
    return bool(ok)


@pytest.mark.parametrize("name", list(MASK_MUTATIONS))
def test_mask_mutant_is_caught(tmp_path, name):
    old, new = MASK_MUTATIONS[name]
    attention = build_mutant(tmp_path, name, old, new)
    assert not masked_pins_pass(attention.masked), f"mutation {name!r} was not detected by any pin"


def test_unmutated_oracle_passes_the_masked_pins(tmp_path):
    attention = build_mutant(tmp_path, "none", "int oracle_max_threads(void)", "int oracle_max_threads(void)")
    assert masked_pins_pass(attention.masked)


def bwd_pins_pass(bwd):
    """Finite differences of an independent fp64 forward, causal and not."""
    from tests.test_oracle_bwd import finite_diff
    ok = True
    for causal, seed in ((False, 30), (True, 31)):
        Q, K, V = fi.make_qkv(1, 2, 4, 5, 8, seed=seed)
        dO = fi.make_qkv(1, 2, 4, 1, 8, seed=seed + 1)[0]
        dQ, dK, dV, _, _ = bwd(Q, K, V, dO, 0.4, causal)
        gQ, gK, gV = finite_diff(widen(Q), widen(K), widen(V), widen(dO), np.float64(np.float32(0.4)), causal, None)
        ok &= all(np.allclose(a, b, rtol=0, atol=2e-7) for a, b in ((dQ, gQ), (dK, gK), (dV, gV)))
    return bool(ok)


def test_unmutated_oracle_passes_the_backward_pins(tmp_path):
    attention = build_mutant(tmp_path, "none", "int oracle_max_threads(void)", "int oracle_max_threads(void)")
    assert bwd_pins_pass(attention.bwd)


@pytest.mark.parametrize("name", list(BWD_MUTATIONS))
def test_backward_mutant_is_caught(tmp_path, name):
    old, new = BWD_MUTATIONS[name]
    attention = build_mutant(tmp_path, name, old, new)
    assert not bwd_pins_pass(attention.bwd), f"mutation {name!r} was not detected by any pin"
