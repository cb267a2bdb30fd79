"""Independent brute-force attention for tiny inputs (pure Python).

Used only to pin the fp64 oracle.  It shares nothing with the oracle beyond
the definition of the function both compute ("FlashAttention'ı Anlamak
Bölüm 1", section 0.2: S = Q K^T * scale, P = softmax_row(S), O = P V) and
takes a different route to it:

  * each dot product is exact before its one final rounding: a bf16 value has
    8 significant bits, so every product has at most 16 and is exact in a
    Python float, and ``math.fsum`` returns the correctly rounded sum;
  * the exponentials are taken of the *unshifted* logits (no running or
    row maximum at all), so the inputs must keep |s| small;
  * the sums over keys use ``math.fsum``.
"""
import math

import numpy as np


def _widen(bits):
    b = np.asarray(bits, dtype=np.uint16)
    return (b.astype(np.uint32) << np.uint32(16)).view(np.float32).astype(np.float64)


def attention(Q, K, V, scale, causal=False, bias=None):
    """Optional mask/bias term: ``causal`` drops key j for query i when
    j > i + (Nk - Nq); ``bias`` (float32, broadcastable to [B, H, Nq, Nk]) is
    added to the scaled logits, and a key whose bias is -inf is dropped.  A
    row left with no key gives O = 0 and LSE = -inf."""
    B, H, Nq, d = Q.shape
    Nk = K.shape[2]
    dv = V.shape[3]
    q, k, v = _widen(Q).tolist(), _widen(K).tolist(), _widen(V).tolist()
    bb = None if bias is None else np.broadcast_to(np.asarray(bias, np.float32), (B, H, Nq, Nk)).astype(np.float64)
    sigma = float(np.float32(scale))
    O = np.zeros((B, H, Nq, dv))
    LSE = np.zeros((B, H, Nq))
    for b in range(B):
        for h in range(H):
            for i in range(Nq):
                qi = q[b][h][i]
                keys, w = [], []
                for j in range(Nk):
                    if causal and j > i + (Nk - Nq):
                        continue
                    extra = 0.0 if bb is None else float(bb[b, h, i, j])
                    if extra == -math.inf:
                        continue
                    dot = math.fsum(qi[c] * k[b][h][j][c] for c in range(d))
                    keys.append(j)
                    w.append(math.exp(sigma * dot + extra))
                if not keys:
                    LSE[b, h, i] = -math.inf
                    continue
                l = math.fsum(w)
                for c in range(dv):
                    O[b, h, i, c] = math.fsum(wj * v[b][h][j][c] for wj, j in zip(w, keys)) / l
                LSE[b, h, i] = math.log(l)
    return O, LSE
