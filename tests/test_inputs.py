"""The seeded input generator (CPU only)."""
import numpy as np
import torch

import fa06_inputs as fi


def test_deterministic_per_seed():
    a = fi.make_qkv(1, 2, 33, 17, 128, seed=5)
    b = fi.make_qkv(1, 2, 33, 17, 128, seed=5)
    c = fi.make_qkv(1, 2, 33, 17, 128, seed=6)
    for x, y in zip(a, b):
        assert np.array_equal(x, y)
    assert not np.array_equal(a[0], c[0])


def test_bf16_rounding_matches_torch():
    rng = np.random.default_rng(0)
    x = np.concatenate([rng.standard_normal(200000).astype(np.float32) * s for s in (1e-3, 1, 50, 1e5)])
    # ties: values exactly halfway between two bf16 numbers
    ties = ((np.arange(1, 2000, dtype=np.uint32) << 16) | 0x8000).view(np.float32)
    x = np.concatenate([x, ties, -ties, np.array([0.0, -0.0, 1.0, 65504.0], np.float32)])
    mine = fi.f32_to_bf16_bits(x)
    ref = torch.from_numpy(x).to(torch.bfloat16).view(torch.int16).numpy().view(np.uint16)
    assert np.array_equal(mine, ref)
    assert np.array_equal(fi.bf16_bits_to_f32(mine), torch.from_numpy(x).to(torch.bfloat16).float().numpy())


def test_offset_rows_per_head():
    w = fi.WORKLOADS["b1_h16_n16384_koffset"]
    assert fi.offset_row_count(w.Nk, w.offset_frac) == 164
    # small analogue of the offset workload: exactly round(1% of Nk) rows carry +8
    Q, K, V = fi.make_qkv(1, 3, 8, 1000, 16, seed=9, k_scale=4.0, offset_frac=0.01, offset=8.0)
    kf = fi.bf16_bits_to_f32(K)
    for h in range(3):
        shifted = (kf[0, h].mean(axis=1) > 4.0).sum()
        assert shifted == 10


def test_workload_table():
    w = fi.WORKLOADS
    assert [(x.B, x.H, x.Nq, x.Nk, x.d, x.d_v) for x in w.values()] == [
        (1, 1, 256, 256, 128, 128), (1, 8, 4096, 8192, 128, 128), (4, 16, 4096, 4096, 128, 128),
        (2, 16, 8192, 8192, 128, 128), (1, 16, 16384, 16384, 128, 128), (2, 32, 8192, 8192, 64, 64),
        (2, 8, 8192, 8192, 256, 256), (2, 16, 8192, 8192, 192, 128)]
    assert w["rtx5090_q4096_kv8192"].flops == 137438953472
    # 2 B H Nq Nk (d + d_v): Q K^T over 192, P V over 128
    assert w["b2_h16_n8192_d192_dv128"].flops == 2 * 2 * 16 * 8192 * 8192 * (192 + 128)
    Q, K, V = fi.make_workload(fi.Workload("t", 1, 2, 3, 5, d=192, seed=1, dv=128))
    assert Q.shape == (1, 2, 3, 192) and K.shape == (1, 2, 5, 192) and V.shape == (1, 2, 5, 128)
    assert abs(w["tiny_256"].scale - 0.08838834764831845) < 1e-8


def test_sample_rows_cover_head_edges():
    r = fi.sample_rows(2, 3, 100, 50, seed=1)
    assert len(set(r)) == len(r) and r.min() >= 0 and r.max() < 600
    for bh in range(6):
        assert bh * 100 in r and bh * 100 + 99 in r
