"""MXFP8 encoding for the oracle (numpy, fp64).

TEST INFRASTRUCTURE ONLY (see ``oracle/__init__.py``): used by the tests to
quantize inputs for the MXFP8 attention path and to dequantize them for the
fp64 attention oracle.  It shares nothing with the GPU path.

The pages name MXFP8 attention as the goal of their kernel work ("Flash
Attention на 5090 в CUDA C++", the motivation and "Что дальше") without
defining the format; this module follows the Open Compute Project
microscaling (MX) format definition:

* element type E4M3 (sign, 4 exponent bits with bias 7, 3 mantissa bits;
  exponent 0 encodes subnormals m * 2^-9; the all-ones exponent and mantissa
  pattern is NaN, there is no infinity; largest finite value 448);
* blocks of 32 consecutive elements share one E8M0 scale 2^(s - 127)
  (s = 255 is NaN);
* the shared exponent of a block is floor(log2(max |v|)) - 8 (8 is E4M3's
  largest exponent), clamped to the E8M0 range; an all-zero block uses the
  smallest scale 2^-127;
* each element is v / 2^shared rounded to the nearest E4M3 value, ties to
  the even code, magnitudes above 448 saturate to 448 (the format leaves
  overflow handling to the implementation; saturation is the reading taken).
"""
from __future__ import annotations

import numpy as np

BLOCK = 32
E4M3_MAX = 448.0
E4M3_EMAX = 8          # exponent of the largest E4M3 binade (2^8 * 1.75 = 448)
E4M3_NAN = 0x7F


def _decode_table() -> np.ndarray:
    t = np.empty(256, dtype=np.float64)
    for code in range(256):
        sign = -1.0 if code & 0x80 else 1.0
        e = (code >> 3) & 0xF
        m = code & 0x7
        if e == 0xF and m == 0x7:
            t[code] = np.nan
        elif e == 0:
            t[code] = sign * m * 2.0 ** -9
        else:
            t[code] = sign * (1.0 + m / 8.0) * 2.0 ** (e - 7)
    return t


E4M3_VALUES = _decode_table()
# non-negative finite values in code order 0x00..0x7E (increasing)
_POS = E4M3_VALUES[:0x7F]


def e4m3_decode(codes: np.ndarray) -> np.ndarray:
    return E4M3_VALUES[np.asarray(codes, dtype=np.uint8)]


def e4m3_encode(x: np.ndarray) -> np.ndarray:
    """Round to the nearest E4M3 value (ties to the even code), saturating."""
    x = np.asarray(x, dtype=np.float64)
    a = np.minimum(np.abs(x), E4M3_MAX)
    hi = np.clip(np.searchsorted(_POS, a, side="left"), 0, len(_POS) - 1)
    lo = np.maximum(hi - 1, 0)
    dlo = a - _POS[lo]
    dhi = _POS[hi] - a
    pick_hi = (dhi < dlo) | ((dhi == dlo) & (hi % 2 == 0))
    code = np.where(pick_hi, hi, lo).astype(np.uint8)
    code = np.where(np.signbit(x), code | 0x80, code).astype(np.uint8)
    return np.where(np.isnan(x), np.uint8(E4M3_NAN), code).astype(np.uint8)


def e8m0_decode(s: np.ndarray) -> np.ndarray:
    s = np.asarray(s, dtype=np.int64)
    return np.where(s == 255, np.nan, np.ldexp(1.0, s - 127))


def mx_quantize(x: np.ndarray):
    """Blocks of 32 along the last axis (its length a multiple of 32).

    Returns (elements uint8 [..., n], scales uint8 [..., n/32])."""
    x = np.asarray(x, dtype=np.float64)
    n = x.shape[-1]
    if n % BLOCK:
        raise ValueError(f"last axis ({n}) must be a multiple of {BLOCK}")
    blocks = x.reshape(*x.shape[:-1], n // BLOCK, BLOCK)
    amax = np.abs(blocks).max(axis=-1)
    # floor(log2 amax) exactly: amax = m * 2^e with m in [0.5, 1)
    _, e = np.frexp(np.where(amax > 0, amax, 1.0))
    shared = np.where(amax > 0, e.astype(np.int64) - 1 - E4M3_EMAX, -127)
    shared = np.clip(shared, -127, 127).astype(np.int64)
    elems = e4m3_encode(blocks / np.ldexp(1.0, shared)[..., None])
    return elems.reshape(x.shape), (shared + 127).astype(np.uint8)


def mx_dequantize(elems: np.ndarray, scales: np.ndarray) -> np.ndarray:
    """Exact values element * 2^(scale - 127), blocks of 32 along the last axis."""
    e = e4m3_decode(elems)
    n = e.shape[-1]
    blocks = e.reshape(*e.shape[:-1], n // BLOCK, BLOCK)
    return (blocks * e8m0_decode(scales)[..., None]).reshape(e.shape)


def as_bf16_bits(values: np.ndarray) -> np.ndarray:
    """Exact bf16 bits of values that bf16 represents (E4M3 element times a
    power of two within bf16's range); raises if any value would round."""
    f = np.asarray(values, dtype=np.float32)
    if not np.array_equal(f.astype(np.float64), np.asarray(values, dtype=np.float64), equal_nan=True):
        raise ValueError("value not exact in float32")
    bits = f.view(np.uint32)
    if np.any(bits & 0xFFFF):
        raise ValueError("value not exact in bf16")
    return (bits >> 16).astype(np.uint16)


def quantize_attention_inputs(Q: np.ndarray, K: np.ndarray, V: np.ndarray, ldv: int | None = None):
    """MXFP8 encodings of float Q [B,H,Nq,d], K [B,H,Nk,d] (blocks along d)
    and V (blocks along the keys: V^T [B,H,dv,ldv], keys padded with zeros
    to ldv, a multiple of 32).  Returns (q8, qs, k8, ks, vt8, vs) and the
    exact bf16 bits of the dequantized Q, K and V for the attention oracle."""
    Nk = K.shape[2]
    ldv = Nk if ldv is None else ldv
    q8, qs = mx_quantize(Q)
    k8, ks = mx_quantize(K)
    Vt = np.zeros((*V.shape[:2], V.shape[3], ldv), dtype=np.float64)
    Vt[..., :Nk] = np.swapaxes(np.asarray(V, dtype=np.float64), -1, -2)
    vt8, vs = mx_quantize(Vt)
    Qd = mx_dequantize(q8, qs)
    Kd = mx_dequantize(k8, ks)
    Vd = np.swapaxes(mx_dequantize(vt8, vs)[..., :Nk], -1, -2)
    return (q8, qs, k8, ks, vt8, vs), (as_bf16_bits(Qd), as_bf16_bits(Kd), as_bf16_bits(np.ascontiguousarray(Vd)))
