"""GPU parity of the MXFP8 path: the encoders bit for bit against the
oracle's MX encoding, and MXFP8 attention against the fp64 oracle on the
exactly dequantized inputs.

Attention gates (derivation): S is exact up to fp32 summation (E4M3
products are exact, the block scales are powers of two), so the LSE keeps
the bf16 path's 1e-3 gate -- the row sum uses the unrounded fp32 P.  The
kernel rounds each probability to E4M3 before P V, in a frame where the
row's largest weight lies in [1, 256] (the lazily raised running max).
Round to nearest moves a normal E4M3 value by at most 2^-4 of itself and a
subnormal one (below 2^-6) by at most 2^-10; after dividing by the row sum
this is at most max(2^-4 P_ij, 2^-10 max_k P_ik) on each normalised weight
P_ij, and 0 for a hidden key.  So, elementwise,
    |dO_ic| <= sum_j max(2^-4 P_ij, 2^-10 max_k P_ik) |v_jc| + 2^-8 |O_ic|,
the last term for the bf16 output rounding (2^-9) and fp32 accumulation;
the tests evaluate this bound in numpy from the dequantized inputs and
require every element within it.  With the rounding error spread uniformly
over +-2^-4 the expected normwise error is 2^-4/sqrt(3) ~ 3.6e-2 of |O| when
the values are independent of the weights; the normwise gate is 6e-2.
"""
import math

import numpy as np
import pytest

import fa06_inputs as fi
import oracle
from oracle import mx
from tests.gpu_util import MAX_ABS_LSE, o_to_f64, say

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128)


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_06_amd as m
    m.load_library()
    return m


def bf16_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def u8_dev(a):
    import torch
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.uint8)).cuda()


def widen(bits):
    return fi.bf16_bits_to_f32(bits).astype(np.float64)


def spread_bits(shape, seed):
    """bf16 values over many binades, with exact ties of the E4M3 grid,
    all-zero blocks and signed zeros."""
    rng = np.random.default_rng(seed)
    x = rng.standard_normal(shape).astype(np.float32)
    x *= np.exp2(rng.integers(-40, 40, size=shape[:-1] + (shape[-1] // 32,))).repeat(32, axis=-1).astype(np.float32)
    flat = x.reshape(-1, 32)
    flat[::7] = 0.0                                        # zero blocks
    flat[1::7, 0] = -0.0
    ties = (1.0 + (2 * rng.integers(0, 8, flat[2::7].shape) + 1) / 16.0) * np.exp2(rng.integers(-3, 3, flat[2::7].shape))
    flat[2::7] = ties.astype(np.float32)                   # midpoints of the E4M3 grid at the block scale
    flat[3::7, 5] = 300.0 * np.abs(flat[3::7]).max(axis=1)  # one large value per block: the rest go subnormal
    return fi.f32_to_bf16_bits(x)


@pytest.mark.parametrize("N", [1, 96, 300])
def test_quantize_rows_bit_exact(fa, N):
    import torch
    say(f"case mx quantize rows N={N}")
    X = spread_bits((2, 3, N, 128), seed=500 + N)
    ld = N + 17
    e, s = fa.mxfp8_quantize_rows(bf16_dev(X), ld=ld)
    torch.cuda.synchronize()
    qe, qs = mx.mx_quantize(widen(X))
    assert np.array_equal(e.cpu().numpy(), qe)
    assert np.array_equal(s.cpu().numpy()[:, :, :N], qs)


@pytest.mark.parametrize("Nk", [1, 64, 200, 513])
def test_quantize_vt_bit_exact(fa, Nk):
    import torch
    say(f"case mx quantize V^T Nk={Nk}")
    V = spread_bits((1, 2, Nk, 128), seed=600 + Nk)
    ldv = (Nk + 63) // 64 * 64
    vt, vs = fa.mxfp8_quantize_vt(bf16_dev(V), ldv=ldv)
    torch.cuda.synchronize()
    Vt = np.zeros((1, 2, 128, ldv))
    Vt[..., :Nk] = np.swapaxes(widen(V), -1, -2)
    qe, qs = mx.mx_quantize(Vt)
    assert np.array_equal(vt.cpu().numpy(), qe)
    assert np.array_equal(vs.cpu().numpy(), np.swapaxes(qs, -1, -2))


def mx_case(B, H, Nq, Nk, seed, **kw):
    """Oracle-side MXFP8 encodings of seeded Q, K, V and the bf16 bits of
    their exact dequantized values."""
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed, **kw)
    ldv = (Nk + 63) // 64 * 64
    (q8, qs, k8, ks, vt8, vs), (Qd, Kd, Vd) = mx.quantize_attention_inputs(widen(Q), widen(K), widen(V), ldv=ldv)
    ks_pad = np.zeros((B, H, ldv, 4), np.uint8)
    ks_pad[:, :, :Nk] = ks
    dev = (u8_dev(q8), u8_dev(qs), u8_dev(k8), u8_dev(ks_pad), u8_dev(vt8), u8_dev(np.swapaxes(vs, -1, -2)))
    return dev, (Qd, Kd, Vd)


def probs64(Qd, Kd, scale, causal, rows=None):
    """Normalised attention weights in fp64 (numpy), [.., Nq or n, Nk], 0 on hidden keys."""
    Q, K = widen(Qd), widen(Kd)
    B, H, Nq, _ = Q.shape
    Nk = K.shape[2]
    if rows is not None:
        bh, i = rows // Nq, rows % Nq
        S = np.einsum("nd,nkd->nk", Q.reshape(-1, 128)[rows], K.reshape(B * H, Nk, 128)[bh]) * np.float32(scale)
        vis = np.ones(S.shape, bool) if not causal else (np.arange(Nk)[None, :] <= (i + Nk - Nq)[:, None])
    else:
        S = (Q @ np.swapaxes(K, -1, -2)) * np.float64(np.float32(scale))
        vis = np.ones(S.shape, bool) if not causal else np.broadcast_to(
            np.arange(Nk)[None, :] <= (np.arange(Nq)[:, None] + Nk - Nq), S.shape)
    S = np.where(vis, S, -np.inf)
    m = S.max(axis=-1, keepdims=True)
    m = np.where(np.isfinite(m), m, 0.0)
    E = np.where(vis, np.exp(S - m), 0.0)
    l = E.sum(axis=-1, keepdims=True)
    return np.where(l > 0, E / np.where(l > 0, l, 1.0), 0.0), vis


def rounding_bound(P, vis, Vabs, Oref):
    """sum_j max(2^-4 P_ij, 2^-10 max_k P_ik) |v_jc| + 2^-8 |O_ic|."""
    W = np.where(vis, np.maximum(2.0 ** -4 * P, 2.0 ** -10 * P.max(axis=-1, keepdims=True)), 0.0)
    return W @ Vabs + 2.0 ** -8 * np.abs(Oref) + 1e-6


def gates(Og, Lg, Oo, Lo, bound, label):
    dO = np.abs(Og - Oo)
    rel = float(np.sqrt((dO ** 2).sum() / (Oo ** 2).sum())) if (Oo ** 2).sum() > 0 else float(dO.max())
    worst = float((dO / bound).max())
    dL = float(np.abs(Lg - Lo).max()) if Lg.size else 0.0
    say(f"  {label}: rel_norm={rel:.3e} max_dO={dO.max():.3e} worst/bound={worst:.3f} max_dLSE={dL:.2e}")
    assert np.all(np.isfinite(Og)) and np.all(np.isfinite(Lg))
    assert rel <= 6e-2, rel
    assert worst <= 1.0, worst
    assert dL <= MAX_ABS_LSE, dL


def check_mx(Og, Lg, Qd, Kd, Vd, scale, causal, label):
    Oo, Lo = oracle.attention_masked(Qd, Kd, Vd, scale, causal=causal)
    P, vis = probs64(Qd, Kd, scale, causal)
    bound = rounding_bound(P, vis, np.abs(widen(Vd)), Oo)
    none = np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), none)
    assert np.all(Og[none] == 0)
    gates(Og[~none], Lg[~none], Oo[~none], Lo[~none], bound[~none], label)


MX_CASES = [
    # B, H, Nq, Nk, causal, seed, note
    (1, 2, 256, 256, False, 700, "tile aligned"),
    (2, 1, 200, 333, False, 701, "ragged Nq and Nk"),
    (1, 2, 256, 256, True, 702, "causal"),
    (1, 1, 300, 130, True, 703, "causal, Nq > Nk: rows that see no key"),
    (1, 1, 129, 65, True, 704, "one row / key past a tile"),
    (1, 2, 1, 700, False, 705, "one query"),
    (1, 1, 70, 1, False, 706, "one key"),
    # grids of >= 256 workgroups of 256 rows: the 8-wave kernel
    (2, 128, 300, 520, False, 720, "8 waves: ragged q tile (44 rows), ragged keys"),
    (1, 256, 256, 1000, False, 721, "8 waves: six segmented iteration pairs, 40-key tail"),
    (2, 128, 512, 512, True, 722, "8 waves: causal"),
    # fewer than 256 workgroups of 256 rows, at least 256 of 128, >= 1024 keys:
    # two key groups of 4 waves per workgroup, merged in LDS
    (1, 128, 256, 1024, False, 730, "key groups: 8 tiles each"),
    (1, 128, 200, 1087, False, 731, "key groups: ragged 17th tile, the second group's 9th past the keys"),
    (1, 128, 256, 1100, True, 732, "key groups, causal"),
    (1, 32, 1280, 1024, True, 733, "key groups, causal, Nq > Nk: whole q-tiles see no key"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,causal,seed,note", MX_CASES)
def test_mxfp8_attention_full_compare(fa, B, H, Nq, Nk, causal, seed, note):
    import torch
    say(f"case mxfp8 B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} seed={seed} ({note})")
    dev, (Qd, Kd, Vd) = mx_case(B, H, Nq, Nk, seed)
    o, lse = fa.fa_fwd_mxfp8(*dev, Nk, scale=SCALE, causal=causal)
    torch.cuda.synchronize()
    check_mx(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Qd, Kd, Vd, SCALE, causal, note)


@pytest.mark.parametrize("scale,note", [(-0.09, "negative scale"), (0.0, "zero scale"), (0.3, "large scale")])
def test_mxfp8_scale_variants(fa, scale, note):
    import torch
    say(f"case mxfp8 scale={scale}")
    dev, (Qd, Kd, Vd) = mx_case(1, 2, 190, 260, 710)
    for causal in (False, True):
        o, lse = fa.fa_fwd_mxfp8(*dev, 260, scale=scale, causal=causal)
        torch.cuda.synchronize()
        check_mx(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Qd, Kd, Vd, scale, causal,
                 f"{note} causal={causal}")


@pytest.mark.parametrize("scale,note", [(-0.09, "negative scale"), (0.0, "zero scale")])
def test_mxfp8_key_group_scales(fa, scale, note):
    import torch
    say(f"case mxfp8 key groups B=1 H=128 Nq=256 Nk=1100 scale={scale} ({note})")
    dev, (Qd, Kd, Vd) = mx_case(1, 128, 256, 1100, 734)
    for causal in (False, True):
        o, lse = fa.fa_fwd_mxfp8(*dev, 1100, scale=scale, causal=causal)
        torch.cuda.synchronize()
        check_mx(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Qd, Kd, Vd, scale, causal,
                 f"key groups {note} causal={causal}")


@pytest.mark.parametrize("scale,note", [(-0.09, "negative scale"), (0.0, "zero scale")])
def test_mxfp8_eight_wave_scales(fa, scale, note):
    import torch
    say(f"case mxfp8 8-wave B=1 H=256 Nq=256 Nk=520 scale={scale} ({note})")
    dev, (Qd, Kd, Vd) = mx_case(1, 256, 256, 520, 724)
    for causal in (False, True):
        o, lse = fa.fa_fwd_mxfp8(*dev, 520, scale=scale, causal=causal)
        torch.cuda.synchronize()
        check_mx(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Qd, Kd, Vd, scale, causal,
                 f"8-wave {note} causal={causal}")


def test_mxfp8_offset_keys(fa):
    import torch
    say("case mxfp8 on the offset-key recipe, B=1 H=2 N=1024")
    dev, (Qd, Kd, Vd) = mx_case(1, 2, 1024, 1024, 711, k_scale=4.0, offset_frac=0.01, offset=8.0)
    o, lse = fa.fa_fwd_mxfp8(*dev, 1024, scale=SCALE)
    torch.cuda.synchronize()
    check_mx(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Qd, Kd, Vd, SCALE, False, "offset keys")


def test_mxfp8_offset_keys_eight_waves(fa):
    import torch
    say("case mxfp8 on the offset-key recipe with 8-wave workgroups, B=1 H=256 Nq=256 Nk=1024")
    dev, (Qd, Kd, Vd) = mx_case(1, 256, 256, 1024, 723, k_scale=4.0, offset_frac=0.01, offset=8.0)
    o, lse = fa.fa_fwd_mxfp8(*dev, 1024, scale=SCALE)
    torch.cuda.synchronize()
    check_mx(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Qd, Kd, Vd, SCALE, False, "offset keys, 8 waves")


def test_mxfp8_end_to_end_with_gpu_quantizers(fa):
    """bf16 q, k, v -> GPU encoders -> MXFP8 attention, against the oracle on
    the oracle's own encoding of the same bf16 values."""
    import torch
    say("case mxfp8 end to end: GPU quantizers + attention, B=2 H=2 N=500")
    Q, K, V = fi.make_qkv(2, 2, 500, 500, 128, seed=712)
    o, lse = fa.fa_fwd_mxfp8(*fa.mxfp8_inputs(bf16_dev(Q), bf16_dev(K), bf16_dev(V)), scale=SCALE)
    torch.cuda.synchronize()
    _, (Qd, Kd, Vd) = mx.quantize_attention_inputs(widen(Q), widen(K), widen(V), ldv=512)
    check_mx(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Qd, Kd, Vd, SCALE, False, "end to end")


def test_mxfp8_workload_sampled(fa):
    import torch
    w = fi.WORKLOADS["b2_h16_n8192"]
    say("case mxfp8 workload b2_h16_n8192 (sampled rows)")
    Q, K, V = fi.make_workload(w)
    o, lse = fa.fa_fwd_mxfp8(*fa.mxfp8_inputs(bf16_dev(Q), bf16_dev(K), bf16_dev(V)), scale=w.scale)
    torch.cuda.synchronize()
    _, (Qd, Kd, Vd) = mx.quantize_attention_inputs(widen(Q), widen(K), widen(V), ldv=w.Nk)
    rows = fi.sample_rows(w.B, w.H, w.Nq, 64, seed=w.seed)
    Oo, Lo = oracle.attention_rows(Qd, Kd, Vd, w.scale, rows)
    P, vis = probs64(Qd, Kd, w.scale, False, rows=rows)
    Vabs = np.abs(widen(Vd)).reshape(w.B * w.H, w.Nk, 128)[rows // w.Nq]
    bound = np.einsum("nk,nkd->nd", np.where(vis, np.maximum(2.0 ** -4 * P, 2.0 ** -10 * P.max(-1, keepdims=True)), 0.0),
                      Vabs) + 2.0 ** -8 * np.abs(Oo) + 1e-6
    idx = torch.from_numpy(rows).cuda()
    Og = o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64)
    Lg = lse.view(-1)[idx].cpu().numpy().astype(np.float64)
    gates(Og, Lg, Oo, Lo, bound, "workload b2_h16_n8192 (sampled)")
