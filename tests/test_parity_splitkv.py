"""GPU parity of the key-split forward (fa_fwd_splitkv) against the fp64
oracle.  Each range of keys is attended to separately and the ranges are
merged by the online-softmax recurrence ("FlashAttention'ı Anlamak Bölüm 1",
section 0); the result must meet the same gates as the one-pass forward,
including rows whose range sees no key (causal), -inf bias entries, every
head-size pair and ragged last ranges."""
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


def compare(fa, Q, K, V, scale, causal, n_splits, label, bias=None):
    import torch
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=scale, causal=causal, bias=bt, n_splits=n_splits)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attention_masked(Q, K, V, scale, causal=causal, bias=bias)
    Og, Lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    none = np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), none), label
    assert np.all(Og[none] == 0), label
    check_parity(Og[~none], Lg[~none], Oo[~none], Lo[~none], label)


CASES = [
    # d, d_v, B, H, Nq, Nk, causal, n_splits, seed, note
    (128, 128, 1, 2, 256, 1000, False, 3, 500, "three ranges, ragged last"),
    (128, 128, 2, 1, 200, 4096, False, 0, 501, "automatic plan"),
    (128, 128, 1, 2, 130, 700, True, 4, 502, "causal, Nk > Nq"),
    (128, 128, 1, 1, 640, 300, True, 3, 503, "causal, Nq > Nk: ranges past the diagonal of a q-tile"),
    (128, 128, 1, 1, 1, 5000, False, 7, 504, "one query row"),
    (128, 128, 1, 1, 64, 64, False, 2, 505, "one tile: the request is cut to one range"),
    (128, 128, 1, 1, 129, 4097, False, 1000, 506, "one range per 64 keys"),
    (64, 64, 1, 2, 190, 900, True, 3, 507, "head size 64"),
    (256, 256, 1, 2, 190, 900, False, 3, 508, "head size 256"),
    (192, 128, 1, 2, 190, 900, True, 3, 509, "head sizes 192 / 128"),
]


@pytest.mark.parametrize("d,dv,B,H,Nq,Nk,causal,n,seed,note", CASES)
def test_split_full_compare(fa, d, dv, B, H, Nq, Nk, causal, n, seed, note):
    used = fa.splitkv_workspace_bytes(B, H, Nq, Nk, dv, n)[1]
    say(f"case split d={d} d_v={dv} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} n={n} -> {used} ranges ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=seed, dv=dv)
    compare(fa, Q, K, V, 1.0 / math.sqrt(d), causal, n, note)


# Key splits whose grid holds at least 256 workgroups of 256 query rows
# (B*H*ceil(Nq/256)*ranges >= 256, no mask, no bias): the ranges run the
# 8-wave head-size-128 kernel with the segmented iteration.
SEG_SPLIT_CASES = [
    # B, H, Nq, Nk, n_splits, seed, scale, kwargs, note
    (1, 8, 4096, 8192, 0, 520, None, {}, "the 5090 benchmark shape, automatic plan (two ranges)"),
    (1, 128, 300, 129, 2, 521, None, {}, "ranges of 128 keys and of 1 key, ragged q tile"),
    (2, 64, 256, 1000, 3, 522, None, {}, "three ranges, ragged last"),
    (1, 128, 256, 2000, 4, 523, -0.07, dict(k_scale=4.0, offset_frac=0.01, offset=8.0),
     "negative scale, large logits (the 16K workload's recipe)"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,n,seed,scale,kw,note", SEG_SPLIT_CASES)
def test_split_eight_wave_full_compare(fa, B, H, Nq, Nk, n, seed, scale, kw, note):
    used = fa.splitkv_workspace_bytes(B, H, Nq, Nk, 128, n)[1]
    assert B * H * ((Nq + 255) // 256) * used >= 256
    say(f"case split 8-wave B={B} H={H} Nq={Nq} Nk={Nk} n={n} -> {used} ranges ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed, **kw)
    compare(fa, Q, K, V, 1.0 / math.sqrt(128) if scale is None else scale, False, n, note)


def test_split_bias_negative_scale_and_offsets(fa):
    say("case split: bias with -inf keys (causal and not), negative scale, offset-key recipe")
    Q, K, V = fi.make_qkv(1, 2, 190, 1100, 128, seed=510, k_scale=4.0, offset_frac=0.02, offset=8.0)
    rng = np.random.default_rng(511)
    bias = (2.0 * rng.standard_normal((1, 2, 190, 1100))).astype(np.float32)
    bias[0, 1, :, 300:] = -np.inf      # the second and third ranges of head 1 see no key
    for causal in (False, True):
        compare(fa, Q, K, V, 1.0 / math.sqrt(128), causal, 3, f"bias causal={causal}", bias=bias)
    compare(fa, Q, K, V, -0.07, False, 3, "negative scale")


def test_split_matches_unsplit_and_reuses_workspace(fa):
    import torch
    say("case split vs one pass on the same inputs; one workspace for two calls")
    Q, K, V = fi.make_qkv(2, 4, 300, 3000, 128, seed=512)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o1, l1 = fa.fa_fwd(q, k, v)
    need, used = fa.splitkv_workspace_bytes(2, 4, 300, 3000, 128, 4)
    ws = torch.empty(need, dtype=torch.uint8, device="cuda")
    o2, l2 = fa.fa_fwd(q, k, v, n_splits=4, workspace=ws)
    o3, l3 = fa.fa_fwd(q, k, v, n_splits=4, workspace=ws)
    torch.cuda.synchronize()
    assert used == 4
    assert torch.equal(o2.view(torch.int16), o3.view(torch.int16)) and torch.equal(l2, l3)
    # the two orders of summation differ by rounding only
    assert float((o1.float() - o2.float()).abs().max()) <= 1e-2
    assert float((l1 - l2).abs().max()) <= 1e-4


@pytest.mark.parametrize("name,causal", [("rtx5090_q4096_kv8192", False), ("rtx5090_q4096_kv8192", True)])
def test_split_workload_sampled(fa, name, causal):
    import torch
    w = fi.WORKLOADS[name]
    used = fa.splitkv_workspace_bytes(w.B, w.H, w.Nq, w.Nk, w.d_v, 0)[1]
    say(f"case split workload {name} causal={causal} (automatic plan: {used} ranges, sampled rows)")
    assert used == 2
    Q, K, V = fi.make_workload(w)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=w.scale, causal=causal, n_splits=0)
    torch.cuda.synchronize()
    rows = fi.sample_rows(w.B, w.H, w.Nq, 192, seed=w.seed + 11)
    Or, Lr = oracle.attention_masked(Q, K, V, w.scale, causal=causal, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check_parity(o.view(-1, w.d_v)[idx].float().cpu().numpy().astype(np.float64),
                 lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr, f"{name} split causal={causal}")


def test_split_long_keys_short_queries_sampled(fa):
    import torch
    B, H, Nq, Nk = 1, 16, 128, 65536
    used = fa.splitkv_workspace_bytes(B, H, Nq, Nk, 128, 0)[1]
    say(f"case split: {H} heads x {Nq} queries against {Nk} keys (automatic plan: {used} ranges)")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=513)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), n_splits=0)
    torch.cuda.synchronize()
    rows = fi.sample_rows(B, H, Nq, 48, seed=514)
    Or, Lr = oracle.attention_rows(Q, K, V, 1.0 / math.sqrt(128), rows)
    idx = torch.from_numpy(rows).cuda()
    check_parity(o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64),
                 lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr, "long keys, short queries")
