"""Execution contract of the C ABI on the GPU: calls on different streams run
concurrently and give the same bits as sequential calls, the launches can be
captured in a HIP graph (through torch.cuda.graph) and replayed, and the
autograd entry point (attention) gives exactly fa_fwd's output and fa_bwd's
gradients.

Every kernel here is deterministic (no atomics), so results are compared
bit for bit.  Graph tests replay several times with eager work and new
input values in between, and check every replay against an eager call on
the same inputs.  No captured call issues a memset or an allocation: the
key-split forward's workspace is allocated before capture."""
import math

import numpy as np
import pytest

import fa06_inputs as fi
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_06_amd as m
    m.load_library()
    return m


def same(a, b):
    import torch
    if a.dtype == torch.bfloat16:
        return torch.equal(a.view(torch.int16), b.view(torch.int16))
    return torch.equal(a, b)


def test_two_streams_match_sequential(fa):
    import torch
    say("case two concurrent streams vs sequential calls")
    ins = [fi.make_qkv(2, 4, 700, 900, 128, seed=s) for s in (600, 601)]
    dev = [tuple(to_dev(x) for x in t) for t in ins]
    ref = [fa.fa_fwd(*d, causal=(i == 1)) for i, d in enumerate(dev)]
    torch.cuda.synchronize()
    s1, s2 = torch.cuda.Stream(), torch.cuda.Stream()   # default priority
    torch.cuda.current_stream().synchronize()
    outs = []
    for _ in range(3):
        with torch.cuda.stream(s1):
            a = fa.fa_fwd(*dev[0])
        with torch.cuda.stream(s2):
            b = fa.fa_fwd(*dev[1], causal=True)
        outs.append((a, b))
    torch.cuda.synchronize()
    for a, b in outs:
        assert same(a[0], ref[0][0]) and same(a[1], ref[0][1])
        assert same(b[0], ref[1][0]) and same(b[1], ref[1][1])


def new_values(t, seed):
    """Fresh bf16 values of t's shape, written into t in place (eager)."""
    import torch
    g = torch.Generator(device=t.device).manual_seed(seed)
    t.copy_(torch.randn(t.shape, generator=g, device=t.device, dtype=torch.float32).to(torch.bfloat16))


def capture(fn):
    import torch
    side = torch.cuda.Stream()
    side.wait_stream(torch.cuda.current_stream())
    with torch.cuda.stream(side):
        fn()   # warm-up outside the graph (caches the device check)
    torch.cuda.current_stream().wait_stream(side)
    torch.cuda.synchronize()
    g = torch.cuda.CUDAGraph()
    with torch.cuda.graph(g):
        fn()
    torch.cuda.synchronize()
    return g


@pytest.mark.parametrize("variant", ["plain", "causal_bias", "split"])
def test_forward_graph_replays(fa, variant):
    import torch
    say(f"case forward captured in a graph: {variant}")
    B, H, Nq, Nk = 1, 4, 300, 2500
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=610)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o = torch.empty((B, H, Nq, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((B, H, Nq), dtype=torch.float32, device="cuda")
    kw = {}
    if variant == "causal_bias":
        kw = dict(causal=True, bias=torch.randn((1, H, 1, Nk), device="cuda", dtype=torch.float32))
    if variant == "split":
        need, used = fa.splitkv_workspace_bytes(B, H, Nq, Nk, 128, 3)
        assert used == 3
        kw = dict(n_splits=3, workspace=torch.empty(need, dtype=torch.uint8, device="cuda"))
    g = capture(lambda: fa.fa_fwd(q, k, v, out=o, lse=lse, **kw))
    for rep in range(4):
        new_values(q, 700 + rep)
        new_values(v, 800 + rep)
        torch.cuda.synchronize()
        g.replay()
        torch.cuda.synchronize()
        o_g, l_g = o.clone(), lse.clone()
        o_e, l_e = fa.fa_fwd(q, k, v, **{kk: vv for kk, vv in kw.items() if kk != "workspace"})
        torch.cuda.synchronize()
        assert same(o_g, o_e) and same(l_g, l_e), f"replay {rep} differs from the eager call"


def test_backward_graph_replays(fa):
    import torch
    say("case backward captured in a graph")
    B, H, Nq, Nk = 1, 2, 333, 400
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=620)
    dO = fi.make_qkv(B, H, Nq, 1, 128, seed=621)[0]
    q, k, v, g_o = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    o, lse = fa.fa_fwd(q, k, v)
    dq, dk, dv = torch.empty_like(q), torch.empty_like(k), torch.empty_like(v)
    delta = torch.empty_like(lse)
    graph = capture(lambda: fa.fa_bwd(q, k, v, o, lse, g_o, dq=dq, dk=dk, dv=dv, delta=delta))
    for rep in range(3):
        new_values(g_o, 900 + rep)
        torch.cuda.synchronize()
        graph.replay()
        torch.cuda.synchronize()
        got = [t.clone() for t in (dq, dk, dv, delta)]
        want = fa.fa_bwd(q, k, v, o, lse, g_o)
        torch.cuda.synchronize()
        for a, b in zip(got, want):
            assert same(a, b), f"backward replay {rep} differs from the eager call"


@pytest.mark.parametrize("d,dv,causal,with_bias", [(128, 128, False, False), (128, 128, True, True),
                                                   (192, 128, True, False), (64, 64, False, True)])
def test_autograd_attention_matches_direct_calls(fa, d, dv, causal, with_bias):
    import torch
    say(f"case autograd attention d={d} d_v={dv} causal={causal} bias={with_bias}")
    Q, K, V = fi.make_qkv(2, 2, 200, 333, d, seed=630, dv=dv)
    q, k, v = (to_dev(x).requires_grad_(True) for x in (Q, K, V))
    bias = torch.randn((1, 2, 1, 333), device="cuda") if with_bias else None
    o = fa.attention(q, k, v, causal=causal, bias=bias)
    # a non-contiguous upstream gradient (a transposed view)
    g = torch.randn((2, 2, dv, 200), device="cuda").to(torch.bfloat16).transpose(2, 3)
    o.backward(g)
    torch.cuda.synchronize()
    qd, kd, vd = (x.detach() for x in (q, k, v))
    o2, lse2 = fa.fa_fwd(qd, kd, vd, causal=causal, bias=bias)
    dq, dk, dv_, _ = fa.fa_bwd(qd, kd, vd, o2, lse2, g.contiguous(), causal=causal, bias=bias)
    torch.cuda.synchronize()
    assert same(o.detach(), o2)
    assert same(q.grad, dq) and same(k.grad, dk) and same(v.grad, dv_)
    with pytest.raises(NotImplementedError):
        fa.attention(qd, kd, vd, bias=torch.zeros((1, 2, 1, 333), device="cuda", requires_grad=True))
