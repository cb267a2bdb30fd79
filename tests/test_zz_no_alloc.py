"""fa_fwd_splitkv_noalloc (through the C ABI) against fa_fwd_splitkv with a
caller workspace, and against the fp64 oracle.

The no-allocation entry point runs the same kernels with the key ranges'
partials in the library's scratch array, so on the same inputs and plan its
outputs must equal the workspace entry point's bit for bit.  Two calls in a
row, the second with a smaller input, show that what the first call left in
the array does not leak into the second.  A plan that needs more than the
array holds is rejected before anything runs.
"""
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


def run_both(fa, B, H, Nq, Nk, d, dv, causal, n_splits, seed):
    import torch
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=seed, dv=dv)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    sc = 1.0 / math.sqrt(d)
    s = torch.cuda.current_stream().cuda_stream
    need, used = fa.splitkv_workspace_bytes(B, H, Nq, Nk, dv, n_splits)
    assert need <= fa.splitkv_noalloc_max_bytes()
    ws = torch.empty(max(need, 16), dtype=torch.uint8, device="cuda")
    o1 = torch.empty((B, H, Nq, dv), dtype=torch.bfloat16, device="cuda")
    l1 = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    o2 = torch.full_like(o1, float("nan"))
    l2 = torch.full_like(l1, float("nan"))
    rc1 = fa.fa_fwd_splitkv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o1.data_ptr(), l1.data_ptr(),
                                B, H, Nq, Nk, d, dv, sc, int(causal), None, 0, 0, 0, n_splits,
                                ws.data_ptr(), need, s)
    rc2 = fa.fa_fwd_splitkv_noalloc_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                                        B, H, Nq, Nk, d, dv, sc, int(causal), None, 0, 0, 0, n_splits, s)
    torch.cuda.synchronize()
    assert rc1 == 0 and rc2 == 0, (rc1, rc2)
    say(f"  ranges {used}, scratch bytes used {need}")
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)), "O differs from the workspace entry point"
    assert torch.equal(l1, l2), "LSE differs from the workspace entry point"
    if causal:
        Oo, Lo = oracle.attention_masked(Q, K, V, sc, causal=True)
    else:
        Oo, Lo = oracle.attention(Q, K, V, sc)
    Og, Lg = o_to_f64(o2), l2.cpu().numpy().astype(np.float64)
    vis = ~np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), ~vis)
    check_parity(Og[vis], Lg[vis], Oo[vis], Lo[vis], f"noalloc B={B} H={H} Nq={Nq} Nk={Nk} d={d}")
    return used


def test_two_calls_second_smaller(fa):
    say("case noalloc: 1x8x512x4096 auto plan, then 1x2x200x1500 causal, 3 ranges")
    assert run_both(fa, 1, 8, 512, 4096, 128, 128, False, 0, seed=301) > 1
    assert run_both(fa, 1, 2, 200, 1500, 128, 128, True, 3, seed=302) == 3


def test_other_head_sizes_and_one_range(fa):
    say("case noalloc: (192, 128) ragged, 5 ranges; head size 64 with one range")
    assert run_both(fa, 2, 2, 130, 2000, 192, 128, False, 5, seed=303) == 5
    assert run_both(fa, 1, 2, 256, 700, 64, 64, False, 1, seed=304) == 1


def test_plan_above_the_scratch_is_rejected(fa):
    import torch
    say("case noalloc: plan above the scratch array")
    B, H, Nq, Nk = 1, 16, 8192, 1024
    need, used = fa.splitkv_workspace_bytes(B, H, Nq, Nk, 128, 2)
    assert need > fa.splitkv_noalloc_max_bytes()
    q = torch.zeros((B, H, Nq, 128), dtype=torch.bfloat16, device="cuda")
    k = torch.zeros((B, H, Nk, 128), dtype=torch.bfloat16, device="cuda")
    o = torch.full((B, H, Nq, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    lse = torch.full((B, H, Nq), 7.0, dtype=torch.float32, device="cuda")
    rc = fa.fa_fwd_splitkv_noalloc_raw(q.data_ptr(), k.data_ptr(), k.data_ptr(), o.data_ptr(), lse.data_ptr(),
                                       B, H, Nq, Nk, 128, 128, 0.088, 0, None, 0, 0, 0, 2,
                                       torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 9 and "scratch" in fa.fa_status_string(rc)
    assert bool((o.float() == 7.0).all()) and bool((lse == 7.0).all()), "a rejected call must not write"
