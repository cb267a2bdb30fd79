"""fp64 CPU attention oracle (ctypes front end for ``fa_oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by the tests, by the smoke check and by the
benchmark's CPU-baseline leg, never by the product path.  It imports nothing
from the GPU package and the GPU package imports nothing from here; the two
share only the seeded inputs.

The arithmetic lives in ``fa_oracle.c``: exact scaled-dot-product attention
as defined in "FlashAttention'ı Anlamak Bölüm 1", section 0.2 "Notasyon"
(score and output equations, with the optional mask/bias term as an fp32
additive bias and/or a causal mask), evaluated row by row in fp64 from the
bf16 input bits.  Outputs: O in fp64 (never rounded to bf16) and the
natural-log log-sum-exp of the scaled (and biased) logits per query row.
The backward pass (dQ, dK, dV of a loss through O, given dO) is the chain
rule of the same equations, also in fp64 (``attention_bwd*``).  ``mx``
holds the MXFP8 (OCP microscaling, E4M3 elements, E8M0 block scales)
encoding used to prepare inputs of the MXFP8 path; attention on MXFP8 data
is this same oracle applied to the exactly dequantized values.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
_SRC = os.path.join(_HERE, "fa_oracle.c")
_LIB_PATH = os.path.join(_HERE, "liboracle.so")

_i64 = ctypes.c_int64
_p = ctypes.c_void_p


def build(verbose: bool = False) -> str:
    """Compile ``liboracle.so`` with gcc + OpenMP (no fast-math, no FMA contraction)."""
    tmp = _LIB_PATH + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-fno-fast-math", "-ffp-contract=off", "-Wall", "-Wextra",
           _SRC, "-o", tmp, "-lm"]
    if verbose:
        print(" ".join(cmd), flush=True)
    subprocess.run(cmd, check=True)
    os.replace(tmp, _LIB_PATH)
    return _LIB_PATH


_lib_handle = None


def _lib():
    global _lib_handle
    if _lib_handle is None:
        if not os.path.exists(_LIB_PATH):
            build()
        lib = ctypes.CDLL(_LIB_PATH)
        lib.oracle_attn_fp64.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                         ctypes.c_float, _p, _p]
        lib.oracle_attn_fp64.restype = ctypes.c_int
        lib.oracle_attn_rows_fp64.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                              ctypes.c_float, _p, _i64, _p, _p]
        lib.oracle_attn_rows_fp64.restype = ctypes.c_int
        lib.oracle_attn_masked_fp64.argtypes = [_p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                                ctypes.c_float, ctypes.c_int, _p, _i64, _i64, _i64,
                                                _p, _i64, _p, _p]
        lib.oracle_attn_masked_fp64.restype = ctypes.c_int
        lib.oracle_attn_bwd_fp64.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                             ctypes.c_float, ctypes.c_int, _p, _i64, _i64, _i64,
                                             _p, _p, _p, _p, _p]
        lib.oracle_attn_bwd_fp64.restype = ctypes.c_int
        lib.oracle_attn_bwd_dq_rows_fp64.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                                     ctypes.c_float, ctypes.c_int, _p, _i64, _i64, _i64,
                                                     _p, _i64, _p]
        lib.oracle_attn_bwd_dq_rows_fp64.restype = ctypes.c_int
        lib.oracle_attn_bwd_dkdv_keys_fp64.argtypes = [_p, _p, _p, _p, _i64, _i64, _i64, _i64, _i64, _i64,
                                                       ctypes.c_float, ctypes.c_int, _p, _i64, _i64, _i64,
                                                       _p, _i64, _p, _p]
        lib.oracle_attn_bwd_dkdv_keys_fp64.restype = ctypes.c_int
        lib.oracle_max_threads.argtypes = []
        lib.oracle_max_threads.restype = ctypes.c_int
        _lib_handle = lib
    return _lib_handle


def _shapes(Q, K, V):
    for name, a in (("Q", Q), ("K", K), ("V", V)):
        if a.dtype != np.uint16 or a.ndim != 4:
            raise TypeError(f"{name} must be a 4-D uint16 array of bf16 bits, got {a.dtype} {a.shape}")
    B, H, Nq, d = Q.shape
    Bk, Hk, Nk, dk = K.shape
    Bv, Hv, Nv, dv = V.shape
    if (Bk, Hk, dk) != (B, H, d) or (Bv, Hv, Nv) != (B, H, Nk):
        raise ValueError(f"shape mismatch Q{Q.shape} K{K.shape} V{V.shape}")
    return B, H, Nq, Nk, d, dv


def attention(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float):
    """Full oracle: returns (O [B,H,Nq,dv] fp64, LSE [B,H,Nq] fp64)."""
    B, H, Nq, Nk, d, dv = _shapes(Q, K, V)
    Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
    O = np.empty((B, H, Nq, dv), dtype=np.float64)
    LSE = np.empty((B, H, Nq), dtype=np.float64)
    rc = _lib().oracle_attn_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data,
                                 B, H, Nq, Nk, d, dv, ctypes.c_float(scale),
                                 O.ctypes.data, LSE.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attn_fp64 failed with code {rc}")
    return O, LSE


def attention_rows(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, rows: np.ndarray):
    """Selected query rows (flat indices into [B*H*Nq]): (O [n,dv], LSE [n])."""
    B, H, Nq, Nk, d, dv = _shapes(Q, K, V)
    Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    n = rows.shape[0]
    O = np.empty((n, dv), dtype=np.float64)
    LSE = np.empty((n,), dtype=np.float64)
    rc = _lib().oracle_attn_rows_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data,
                                      B, H, Nq, Nk, d, dv, ctypes.c_float(scale),
                                      rows.ctypes.data, n, O.ctypes.data, LSE.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attn_rows_fp64 failed with code {rc}")
    return O, LSE


def attention_masked(Q: np.ndarray, K: np.ndarray, V: np.ndarray, scale: float, causal: bool = False,
                     bias: np.ndarray | None = None, rows: np.ndarray | None = None):
    """Attention with the optional mask/bias term.

    ``causal`` hides key j from query i when j > i + (Nk - Nq).  ``bias`` is an
    fp32 array broadcastable to [B, H, Nq, Nk] with unit key stride (zero
    strides broadcast over batch / heads / rows).  Rows that see no key give
    O = 0 and LSE = -inf.  With ``rows`` (flat indices into [B*H*Nq]) the
    results are [n, dv] and [n]; without, [B, H, Nq, dv] and [B, H, Nq].
    """
    B, H, Nq, Nk, d, dv = _shapes(Q, K, V)
    Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
    bias_ptr, sb, sh, sq = None, 0, 0, 0
    if bias is not None:
        bias = np.asarray(bias, dtype=np.float32)
        full = np.broadcast_to(bias, (B, H, Nq, Nk))
        if full.strides[3] != 4:
            bias = np.ascontiguousarray(bias)
            full = np.broadcast_to(bias, (B, H, Nq, Nk))
        sb, sh, sq = (st // 4 for st in full.strides[:3])
        bias_ptr = full.ctypes.data
    if rows is None:
        n = B * H * Nq
        O = np.empty((B, H, Nq, dv), dtype=np.float64)
        LSE = np.empty((B, H, Nq), dtype=np.float64)
        rows_ptr = None
    else:
        rows = np.ascontiguousarray(rows, dtype=np.int64)
        n = rows.shape[0]
        O = np.empty((n, dv), dtype=np.float64)
        LSE = np.empty((n,), dtype=np.float64)
        rows_ptr = rows.ctypes.data
    rc = _lib().oracle_attn_masked_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data,
                                        B, H, Nq, Nk, d, dv, ctypes.c_float(scale), int(bool(causal)),
                                        bias_ptr, sb, sh, sq, rows_ptr, n, O.ctypes.data, LSE.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attn_masked_fp64 failed with code {rc}")
    return O, LSE


def _bias_view(bias, B, H, Nq, Nk):
    if bias is None:
        return None, 0, 0, 0, None
    bias = np.asarray(bias, dtype=np.float32)
    full = np.broadcast_to(bias, (B, H, Nq, Nk))
    if full.strides[3] != 4:
        bias = np.ascontiguousarray(bias)
        full = np.broadcast_to(bias, (B, H, Nq, Nk))
    sb, sh, sq = (st // 4 for st in full.strides[:3])
    return full.ctypes.data, sb, sh, sq, full


def _check_dO(dO, B, H, Nq, dv):
    if dO.dtype != np.uint16 or dO.shape != (B, H, Nq, dv):
        raise TypeError(f"dO must be uint16 bf16 bits of shape {(B, H, Nq, dv)}, got {dO.dtype} {dO.shape}")
    return np.ascontiguousarray(dO)


def attention_bwd(Q, K, V, dO, scale: float, causal: bool = False, bias=None):
    """Gradients of sum(O * dO) for the attention of ``attention_masked``.

    Returns (dQ [B,H,Nq,d], dK [B,H,Nk,d], dV [B,H,Nk,dv], D [B,H,Nq], LSE
    [B,H,Nq]), all fp64; D_i = sum_j P_ij dP_ij.
    """
    B, H, Nq, Nk, d, dv = _shapes(Q, K, V)
    Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
    dO = _check_dO(dO, B, H, Nq, dv)
    bias_ptr, sb, sh, sq, _keep = _bias_view(bias, B, H, Nq, Nk)
    dQ = np.empty((B, H, Nq, d))
    dK = np.empty((B, H, Nk, d))
    dV = np.empty((B, H, Nk, dv))
    D = np.empty((B, H, Nq))
    LSE = np.empty((B, H, Nq))
    rc = _lib().oracle_attn_bwd_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data, dO.ctypes.data,
                                     B, H, Nq, Nk, d, dv, ctypes.c_float(scale), int(bool(causal)),
                                     bias_ptr, sb, sh, sq, dQ.ctypes.data, dK.ctypes.data, dV.ctypes.data,
                                     D.ctypes.data, LSE.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd_fp64 failed with code {rc}")
    return dQ, dK, dV, D, LSE


def attention_bwd_dq_rows(Q, K, V, dO, scale: float, rows, causal: bool = False, bias=None):
    """dQ of selected query rows (flat indices into [B*H*Nq]): [n, d] fp64."""
    B, H, Nq, Nk, d, dv = _shapes(Q, K, V)
    Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
    dO = _check_dO(dO, B, H, Nq, dv)
    bias_ptr, sb, sh, sq, _keep = _bias_view(bias, B, H, Nq, Nk)
    rows = np.ascontiguousarray(rows, dtype=np.int64)
    dQ = np.empty((rows.shape[0], d))
    rc = _lib().oracle_attn_bwd_dq_rows_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data, dO.ctypes.data,
                                             B, H, Nq, Nk, d, dv, ctypes.c_float(scale), int(bool(causal)),
                                             bias_ptr, sb, sh, sq, rows.ctypes.data, rows.shape[0], dQ.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd_dq_rows_fp64 failed with code {rc}")
    return dQ


def attention_bwd_dkdv_keys(Q, K, V, dO, scale: float, keys, causal: bool = False, bias=None):
    """dK and dV of selected keys (flat indices into [B*H*Nk]): ([n, d], [n, dv]) fp64."""
    B, H, Nq, Nk, d, dv = _shapes(Q, K, V)
    Q, K, V = (np.ascontiguousarray(a) for a in (Q, K, V))
    dO = _check_dO(dO, B, H, Nq, dv)
    bias_ptr, sb, sh, sq, _keep = _bias_view(bias, B, H, Nq, Nk)
    keys = np.ascontiguousarray(keys, dtype=np.int64)
    dK = np.empty((keys.shape[0], d))
    dV = np.empty((keys.shape[0], dv))
    rc = _lib().oracle_attn_bwd_dkdv_keys_fp64(Q.ctypes.data, K.ctypes.data, V.ctypes.data, dO.ctypes.data,
                                               B, H, Nq, Nk, d, dv, ctypes.c_float(scale), int(bool(causal)),
                                               bias_ptr, sb, sh, sq, keys.ctypes.data, keys.shape[0],
                                               dK.ctypes.data, dV.ctypes.data)
    if rc != 0:
        raise ValueError(f"oracle_attn_bwd_dkdv_keys_fp64 failed with code {rc}")
    return dK, dV


def max_threads() -> int:
    return int(_lib().oracle_max_threads())
