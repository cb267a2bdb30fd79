"""GPU parity of the forward pass at head sizes 64 and 256 and at query/key
head size 192 with value head size 128 (the head sizes d and d_v are
parameters of the score and output equations of "FlashAttention'ı Anlamak
Bölüm 1", section 0.2), against the fp64 oracle, with the causal mask, the
additive bias, a negative scale, ragged lengths and the longest sequence the
boundary accepts at head sizes 256 and 192."""
import math

import numpy as np
import pytest

import fa06_inputs as fi
import oracle
from tests.gpu_util import check_parity, o_to_f64, say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_06_amd as m
    m.load_library()
    return m


CASES = [
    # d, d_v, B, H, Nq, Nk, causal, seed, note
    (64, 64, 1, 2, 256, 256, False, 400, "tile aligned"),
    (64, 64, 2, 3, 200, 333, False, 401, "ragged"),
    (64, 64, 1, 2, 300, 130, True, 402, "causal, Nq > Nk"),
    (64, 64, 1, 1, 129, 65, True, 403, "causal, one row / key past a tile"),
    # >= 256 workgroups of 256 rows without mask: 8-wave workgroups
    (64, 64, 1, 256, 300, 200, False, 409, "8 waves: ragged q tile (44 rows) and kv tail"),
    (64, 64, 2, 128, 256, 1000, False, 410, "8 waves: seven segmented iteration pairs, ragged kv"),
    (64, 64, 1, 256, 1, 64, False, 411, "8 waves: one query row per head, one kv tile"),
    (256, 256, 1, 2, 256, 256, False, 404, "tile aligned"),
    (256, 256, 2, 3, 200, 333, False, 405, "ragged"),
    (256, 256, 1, 2, 300, 130, True, 406, "causal, Nq > Nk"),
    (256, 256, 1, 1, 640, 640, True, 407, "causal, several q tiles"),
    (256, 256, 1, 1, 33, 7, False, 408, "kv shorter than a tile"),
    (192, 128, 1, 2, 256, 256, False, 430, "tile aligned"),
    (192, 128, 2, 3, 200, 333, False, 431, "ragged"),
    (192, 128, 1, 2, 300, 130, True, 432, "causal, Nq > Nk"),
    (192, 128, 1, 1, 640, 640, True, 433, "causal, several q tiles"),
    (192, 128, 1, 1, 129, 65, True, 434, "causal, one row / key past a tile"),
    (192, 128, 1, 1, 33, 7, False, 435, "kv shorter than a tile"),
    (192, 128, 1, 2, 1, 1000, False, 436, "one query row"),
]


@pytest.mark.parametrize("d,dv,B,H,Nq,Nk,causal,seed,note", CASES)
def test_headdim_full_compare(fa, d, dv, B, H, Nq, Nk, causal, seed, note):
    import torch
    say(f"case d={d} d_v={dv} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=seed, dv=dv)
    assert V.shape[-1] == dv
    sc = 1.0 / math.sqrt(d)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=sc, causal=causal)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attention_masked(Q, K, V, sc, causal=causal)
    Og, Lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    none = np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), none)
    assert np.all(Og[none] == 0)
    check_parity(Og[~none], Lg[~none], Oo[~none], Lo[~none], f"d={d} d_v={dv} {note}")


@pytest.mark.parametrize("d,dv", [(64, 64), (256, 256), (192, 128)])
def test_headdim_bias_and_negative_scale(fa, d, dv):
    import torch
    say(f"case d={d} d_v={dv}: bias (causal and not), negative scale, offset-key recipe")
    Q, K, V = fi.make_qkv(1, 2, 190, 260, d, seed=410 + d, k_scale=4.0, offset_frac=0.02, offset=8.0, dv=dv)
    rng = np.random.default_rng(411 + d)
    bias = (2.0 * rng.standard_normal((1, 2, 190, 260))).astype(np.float32)
    bias[0, 1, :, 100:] = -np.inf
    bt = torch.from_numpy(bias).cuda()
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    for causal in (False, True):
        o, lse = fa.fa_fwd(q, k, v, scale=1.0 / math.sqrt(d), causal=causal, bias=bt)
        torch.cuda.synchronize()
        Oo, Lo = oracle.attention_masked(Q, K, V, 1.0 / math.sqrt(d), causal=causal, bias=bias)
        check_parity(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Oo, Lo, f"d={d} bias causal={causal}")
    o, lse = fa.fa_fwd(q, k, v, scale=-0.07)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attention(Q, K, V, -0.07)
    check_parity(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Oo, Lo, f"d={d} negative scale")


def test_headdim256_max_key_length(fa):
    import torch
    Nk = 1 << 22  # 2^22 rows of 512 bytes: the 2 GiB slice limit at head size 256
    say(f"case d=256 max Nk={Nk}")
    base = fi.make_qkv(1, 1, 1, 4096, 256, seed=420)
    K = np.ascontiguousarray(np.tile(base[1][0, 0], (Nk // 4096, 1)))[None, None]
    V = np.ascontiguousarray(np.tile(base[2][0, 0], (Nk // 4096, 1)))[None, None]
    K[0, 0, -3:] = fi.f32_to_bf16_bits(np.full((3, 256), 0.2, np.float32))
    V[0, 0, -3:] = fi.f32_to_bf16_bits(np.full((3, 256), 3.0, np.float32))
    Q = fi.make_qkv(1, 1, 130, 1, 256, seed=421)[0]
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=1.0 / 16)
    torch.cuda.synchronize()
    rows = np.array([0, 64, 127, 128, 129], dtype=np.int64)
    Or, Lr = oracle.attention_rows(Q, K, V, 1.0 / 16, rows)
    idx = torch.from_numpy(rows).cuda()
    check_parity(o.view(-1, 256)[idx].float().cpu().numpy().astype(np.float64),
                 lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr, "d=256 max Nk")


def test_dv_max_key_length(fa):
    import torch
    Nk = (1 << 30) // 192   # longest K accepted at d = 192: the 2 GiB slice limit
    say(f"case d=192 d_v=128 max Nk={Nk}")
    base = fi.make_qkv(1, 1, 1, 4096, 192, seed=440, dv=128)
    reps = -(-Nk // 4096)
    K = np.ascontiguousarray(np.tile(base[1][0, 0], (reps, 1))[:Nk])[None, None]
    V = np.ascontiguousarray(np.tile(base[2][0, 0], (reps, 1))[:Nk])[None, None]
    K[0, 0, -3:] = fi.f32_to_bf16_bits(np.full((3, 192), 0.2, np.float32))
    V[0, 0, -3:] = fi.f32_to_bf16_bits(np.full((3, 128), 3.0, np.float32))
    Q = fi.make_qkv(1, 1, 130, 1, 192, seed=441)[0]
    sc = 1.0 / math.sqrt(192)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=sc)
    torch.cuda.synchronize()
    assert tuple(o.shape) == (1, 1, 130, 128)
    rows = np.array([0, 64, 127, 128, 129], dtype=np.int64)
    Or, Lr = oracle.attention_rows(Q, K, V, sc, rows)
    idx = torch.from_numpy(rows).cuda()
    check_parity(o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64),
                 lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr, "d=192 d_v=128 max Nk")


def test_dv_workload_causal_sampled(fa):
    import torch
    w = fi.WORKLOADS["b2_h16_n8192_d192_dv128"]
    say(f"case workload {w.name} causal (sampled rows)")
    Q, K, V = fi.make_workload(w)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rows = fi.sample_rows(w.B, w.H, w.Nq, 128, seed=w.seed + 3)
    Or, Lr = oracle.attention_masked(Q, K, V, w.scale, causal=True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check_parity(o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64),
                 lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr, f"{w.name} causal")
