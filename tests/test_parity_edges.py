"""GPU edge cases of fa_fwd: maximum sequence lengths, long ragged K/V,
IEEE propagation of NaN/Inf inputs, and concurrent streams."""
import math

import numpy as np
import pytest

import fa06_inputs as fi
import oracle
from tests.gpu_util import check_parity, o_to_f64, say, to_dev

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


def sampled_parity(fa, Q, K, V, rows, label):
    import torch
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=SCALE)
    torch.cuda.synchronize()
    Or, Lr = oracle.attention_rows(Q, K, V, SCALE, rows)
    idx = torch.from_numpy(rows).cuda()
    og = o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64)
    lg = lse.view(-1)[idx].cpu().numpy().astype(np.float64)
    check_parity(og, lg, Or, Lr, label)
    assert bool(torch.isfinite(lse).all())


def tiled_rows(n_rows, d, seed):
    """n_rows x d bf16 bits built by tiling 4096 random rows (cheap at 2^23 rows)."""
    base = fi.make_qkv(1, 1, 4096, 1, d, seed=seed)[0][0, 0]
    reps = -(-n_rows // 4096)
    return np.ascontiguousarray(np.tile(base, (reps, 1))[:n_rows])[None, None]


def test_max_query_length(fa):
    Nq = fa.FA_MAX_SEQ  # a 2 GiB Q slice: the largest the boundary accepts
    say(f"case max Nq={Nq} Nk=96")
    Q = tiled_rows(Nq, 128, seed=50)
    _, K, V = fi.make_qkv(1, 1, 1, 96, 128, seed=51)
    rows = np.array([0, 1, 4095, 4096, Nq // 2 + 7, Nq - 129, Nq - 128, Nq - 2, Nq - 1], dtype=np.int64)
    sampled_parity(fa, Q, K, V, rows, "max Nq")


def test_max_key_length(fa):
    Nk = fa.FA_MAX_SEQ  # 2 GiB K and V slices
    say(f"case max Nk={Nk} Nq=130")
    K = tiled_rows(Nk, 128, seed=52)
    V = tiled_rows(Nk, 128, seed=53)
    # make the last keys distinct so a dropped tail would show
    K[0, 0, -5:] = fi.f32_to_bf16_bits(np.full((5, 128), 0.25, np.float32))
    V[0, 0, -5:] = fi.f32_to_bf16_bits(np.full((5, 128), 3.0, np.float32))
    Q = fi.make_qkv(1, 1, 130, 1, 128, seed=54)[0]
    rows = np.array([0, 63, 127, 128, 129], dtype=np.int64)
    sampled_parity(fa, Q, K, V, rows, "max Nk")


def test_long_ragged_keys(fa):
    Nk = (1 << 20) + 37
    say(f"case long ragged Nk={Nk}")
    Q, K, V = fi.make_qkv(1, 2, 70, Nk, 128, seed=55, k_scale=2.0, offset_frac=0.001, offset=4.0)
    rows = np.array([0, 33, 69, 70, 101, 139], dtype=np.int64)
    sampled_parity(fa, Q, K, V, rows, "long ragged Nk")


def test_nan_and_inf_propagate(fa):
    import torch
    say("case NaN in K (head 0), Inf in V (head 1), head 2 clean")
    Q, K, V = fi.make_qkv(1, 3, 130, 200, 128, seed=56)
    K[0, 0, 77, 5] = 0x7FC0  # bf16 quiet NaN
    V[0, 1, 150, 9] = 0x7F80  # bf16 +Inf
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=SCALE)
    torch.cuda.synchronize()
    O = o_to_f64(o)[0]            # [head, row, d]
    L = lse.cpu().numpy()[0]      # [head, row]
    # a NaN score enters every row's sum: the whole head is NaN
    assert np.all(np.isnan(O[0])) and np.all(np.isnan(L[0]))
    # an infinite value reaches column 9 of every row (every weight is > 0);
    # the scores, and so the LSE and the other columns, stay finite
    assert np.all(~np.isfinite(O[1, :, 9])) and np.all(np.isfinite(L[1]))
    assert np.all(np.isfinite(np.delete(O[1], 9, axis=1)))
    # the clean head is unaffected
    Oo, Lo = oracle.attention(Q[:, 2:], K[:, 2:], V[:, 2:], SCALE)
    check_parity(O[None, 2:], L[None, 2:].astype(np.float64), Oo, Lo, "clean head next to NaN/Inf heads")


def test_concurrent_streams(fa):
    import torch
    say("case two streams")
    a = [to_dev(x) for x in fi.make_qkv(2, 4, 512, 700, 128, seed=57)]
    b = [to_dev(x) for x in fi.make_qkv(1, 8, 300, 1100, 128, seed=58)]
    ref_a = fa.fa_fwd(*a)
    ref_b = fa.fa_fwd(*b)
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            oa = fa.fa_fwd(*a)
        with torch.cuda.stream(s2):
            ob = fa.fa_fwd(*b)
        outs.append((oa, ob))
    torch.cuda.synchronize()
    for oa, ob in outs:
        assert torch.equal(oa[0].view(torch.int16), ref_a[0].view(torch.int16)) and torch.equal(oa[1], ref_a[1])
        assert torch.equal(ob[0].view(torch.int16), ref_b[0].view(torch.int16)) and torch.equal(ob[1], ref_b[1])
