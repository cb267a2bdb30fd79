"""GPU parity of the attention backward pass (fa_bwd) against the fp64 oracle.

O and LSE come from this library's forward kernel (itself checked against
the oracle elsewhere); the oracle computes the gradients from Q, K, V and dO
alone.  Gates per gradient tensor G in {dQ, dK, dV}, against the unrounded
fp64 oracle:

  * normwise:  ||G_gpu - G_ref||_2 <= 1e-2 * ||G_ref||_2
  * maxwise:   max |G_gpu - G_ref| <= 2e-2 * max |G_ref|

Derivation: the inputs are exact bf16; the kernel rounds P (for dV) and dS
(for dK, dQ) to bf16 before the products and rounds the outputs to bf16,
each a relative error of at most u = 2^-9 ~ 2e-3 per element, independent
across the summed terms, with fp32 accumulation.  D_i is formed from the
bf16-rounded forward output O (another u on a term that is small next to
dP for these inputs).  Three roundings of u bound the normwise error near
3u ~ 6e-3; the gate is 1e-2.  Elementwise, sums with cancellation make the
error of a small entry large relative to that entry, so the elementwise gate
is relative to the tensor's largest entry (2e-2, ten times u).
"""
import math

import numpy as np
import pytest

import fa06_inputs as fi
import oracle
from tests.gpu_util import say, to_dev

pytestmark = pytest.mark.gpu
SCALE = 1.0 / math.sqrt(128)
NORM_TOL = 1e-2
MAX_TOL = 2e-2


@pytest.fixture(scope="module")
def fa():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")
    import flashattention_forward_06_amd as m
    m.load_library()
    return m


def check_grad(name, got, ref, label):
    got = np.asarray(got, dtype=np.float64)
    diff = np.abs(got - ref)
    nref = float(np.sqrt((ref ** 2).sum()))
    mref = float(np.abs(ref).max()) if ref.size else 0.0
    rel = float(np.sqrt((diff ** 2).sum())) / nref if nref > 0 else 0.0
    mx = float(diff.max()) if diff.size else 0.0
    say(f"  {label} {name}: rel_norm={rel:.3e} max_abs={mx:.3e} max_ref={mref:.3e}")
    assert np.all(np.isfinite(got)), f"{name}: non-finite values"
    if nref == 0.0:
        # an exactly-zero reference (one key, zero scale): what remains is
        # fp32 rounding of dP against D (|dP| ~ 10, 2^-24 relative) summed
        # over the rows, far below any nonzero gradient
        assert mx <= 1e-4, (name, mx)
        return
    assert rel <= NORM_TOL, (name, rel)
    assert mx <= MAX_TOL * mref, (name, mx, mref)


def run_bwd(fa, Q, K, V, dO, scale, causal):
    import torch
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    o, lse = fa.fa_fwd(q, k, v, scale=scale, causal=causal)
    dq, dk, dv, delta = fa.fa_bwd(q, k, v, o, lse, g, scale=scale, causal=causal)
    torch.cuda.synchronize()
    return [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)], (q, k, v, g, o, lse)


def make_case(B, H, Nq, Nk, seed, **kw):
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed, **kw)
    dO = fi.make_qkv(B, H, Nq, 1, 128, seed=seed + 5000)[0]
    return Q, K, V, dO


BWD_CASES = [
    # B, H, Nq, Nk, causal, seed, note
    (1, 2, 256, 256, False, 300, "square, tile aligned"),
    (1, 2, 256, 256, True, 301, "square, causal"),
    (2, 1, 200, 333, False, 302, "ragged Nq and Nk"),
    (2, 1, 200, 333, True, 303, "ragged, causal, Nk > Nq"),
    (1, 1, 300, 130, True, 304, "causal, Nq > Nk: leading rows see no key"),
    (1, 2, 1, 700, False, 305, "one query row"),
    (1, 1, 129, 1, False, 306, "one key"),
    (1, 1, 65, 257, True, 307, "one row past a query block, one key past a key tile"),
    (1, 1, 640, 640, True, 308, "several blocks, diagonal through each"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,causal,seed,note", BWD_CASES)
def test_bwd_full_compare(fa, B, H, Nq, Nk, causal, seed, note):
    say(f"case bwd B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} seed={seed} ({note})")
    Q, K, V, dO = make_case(B, H, Nq, Nk, seed)
    (dq, dk, dv), _ = run_bwd(fa, Q, K, V, dO, SCALE, causal)
    rQ, rK, rV, _, L = oracle.attention_bwd(Q, K, V, dO, SCALE, causal=causal)
    for name, a, b in (("dQ", dq, rQ), ("dK", dk, rK), ("dV", dv, rV)):
        check_grad(name, a, b, note)
    # rows that see no key have dQ = 0 exactly
    none = np.isneginf(L)
    assert np.all(dq[none] == 0)


@pytest.mark.parametrize("scale,note", [(-0.2, "negative scale"), (0.0, "zero scale"), (0.35, "large scale")])
def test_bwd_scale_variants(fa, scale, note):
    say(f"case bwd scale={scale} ({note})")
    Q, K, V, dO = make_case(1, 2, 190, 260, 310)
    (dq, dk, dv), _ = run_bwd(fa, Q, K, V, dO, scale, False)
    rQ, rK, rV, _, _ = oracle.attention_bwd(Q, K, V, dO, scale)
    for name, a, b in (("dQ", dq, rQ), ("dK", dk, rK), ("dV", dv, rV)):
        check_grad(name, a, b, note)


def test_bwd_offset_keys(fa):
    say("case bwd on the offset-key recipe (K*4, 1% rows +8), B=1 H=2 N=512, causal and not")
    Q, K, V, dO = make_case(1, 2, 512, 512, 311, k_scale=4.0, offset_frac=0.01, offset=8.0)
    for causal in (False, True):
        (dq, dk, dv), _ = run_bwd(fa, Q, K, V, dO, SCALE, causal)
        rQ, rK, rV, _, _ = oracle.attention_bwd(Q, K, V, dO, SCALE, causal=causal)
        for name, a, b in (("dQ", dq, rQ), ("dK", dk, rK), ("dV", dv, rV)):
            check_grad(name, a, b, f"offset keys causal={causal}")


def test_bwd_no_queries_zeroes_dk_dv(fa):
    import torch
    say("case bwd with Nq = 0: dK = dV = 0")
    Q, K, V, dO = make_case(1, 2, 0, 100, 312)
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    o = torch.empty((1, 2, 0, 128), dtype=torch.bfloat16, device="cuda")
    lse = torch.empty((1, 2, 0), dtype=torch.float32, device="cuda")
    dk = torch.full((1, 2, 100, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    dv = torch.full((1, 2, 100, 128), 7.0, dtype=torch.bfloat16, device="cuda")
    fa.fa_bwd(q, k, v, o, lse, g, dk=dk, dv=dv)
    torch.cuda.synchronize()
    assert bool((dk == 0).all()) and bool((dv == 0).all())


def test_bwd_deterministic_and_delta(fa):
    import torch
    say("case bwd: two calls bit-identical; delta = dO . O")
    Q, K, V, dO = make_case(2, 2, 300, 300, 313)
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    o, lse = fa.fa_fwd(q, k, v)
    r1 = fa.fa_bwd(q, k, v, o, lse, g)
    r2 = fa.fa_bwd(q, k, v, o, lse, g)
    torch.cuda.synchronize()
    for a, b in zip(r1[:3], r2[:3]):
        assert torch.equal(a.view(torch.int16), b.view(torch.int16))
    assert torch.equal(r1[3], r2[3])
    want = (g.float() * o.float()).sum(-1)
    assert torch.allclose(r1[3], want, rtol=1e-5, atol=1e-5)


@pytest.mark.parametrize("name", ["b2_h16_n8192", "rtx5090_q4096_kv8192"])
def test_bwd_workload_sampled(fa, name):
    import torch
    w = fi.WORKLOADS[name]
    say(f"case bwd workload {name} (sampled rows and keys)")
    Q, K, V = fi.make_workload(w)
    dO = fi.make_qkv(w.B, w.H, w.Nq, 1, w.d, seed=w.seed + 5000)[0]
    (dq, dk, dv), _ = run_bwd(fa, Q, K, V, dO, w.scale, False)
    rows = fi.sample_rows(w.B, w.H, w.Nq, 96, seed=w.seed)
    rQ = oracle.attention_bwd_dq_rows(Q, K, V, dO, w.scale, rows)
    # keys from two heads only (each head needs a full pass in the oracle)
    rng = np.random.default_rng(w.seed + 1)
    heads = rng.choice(w.B * w.H, size=2, replace=False)
    keys = np.sort(np.concatenate([h * w.Nk + rng.choice(w.Nk, size=24, replace=False) for h in heads]))
    keys = np.concatenate([keys, [heads[0] * w.Nk, heads[0] * w.Nk + w.Nk - 1]]).astype(np.int64)
    rK, rV = oracle.attention_bwd_dkdv_keys(Q, K, V, dO, w.scale, keys)
    check_grad("dQ rows", dq.reshape(-1, 128)[rows], rQ, name)
    check_grad("dK keys", dk.reshape(-1, 128)[keys], rK, name)
    check_grad("dV keys", dv.reshape(-1, 128)[keys], rV, name)


def make_bias(kind, B, H, Nq, Nk, seed):
    rng = np.random.default_rng(seed)
    if kind == "full":
        b = (2.0 * rng.standard_normal((B, H, Nq, Nk))).astype(np.float32)
        b[0, 0, :, Nk // 3:] = -np.inf         # head 0 sees only its first third of the keys
        b[0, -1, 3, :] = -np.inf               # a row that sees no key: dQ = 0, nothing added to dK, dV
        return b
    if kind == "per_key_large":
        # broadcast over rows; large entries: the zero-padded rows of a ragged
        # last query block would give exp(60) * 0 = inf * 0 without masking.
        # Two such keys share the probability (one alone would take all of
        # it and make dS, hence dQ, vanish to rounding level)
        b = rng.standard_normal((1, H, 1, Nk)).astype(np.float32)
        b[..., 5] = 60.0
        b[..., 77] = 60.0
        return b
    if kind == "alibi":
        i = np.arange(Nq)[:, None] + (Nk - Nq)
        j = np.arange(Nk)[None, :]
        slopes = 2.0 ** -(np.arange(H) + 1.0)
        return (-slopes[:, None, None] * np.abs(i - j))[None].astype(np.float32)
    if kind == "batch_shared":
        return (2.0 * rng.standard_normal((1, H, Nq, Nk))).astype(np.float32)
    if kind == "head_shared":
        return (2.0 * rng.standard_normal((B, 1, Nq, Nk))).astype(np.float32)
    raise ValueError(kind)


BIAS_CASES = [
    # B, H, Nq, Nk, causal, kind, seed, note
    (1, 2, 256, 256, False, "full", 320, "dense bias, tile aligned, -inf keys and an empty row"),
    (2, 2, 200, 333, False, "full", 321, "dense bias, ragged"),
    (1, 2, 200, 333, True, "full", 322, "dense bias, causal, ragged"),
    (1, 2, 200, 130, False, "per_key_large", 323, "per-key bias with +60 entries, ragged last query block"),
    (1, 2, 300, 130, True, "per_key_large", 324, "per-key bias, causal with Nq > Nk"),
    (1, 4, 640, 640, True, "alibi", 325, "ALiBi-like slopes, causal, several blocks"),
    # bias shared by several heads: their workgroups are grouped in the grid
    (3, 2, 300, 333, False, "batch_shared", 326, "[1,H,Nq,Nk] over 3 batches, ragged"),
    (3, 2, 300, 333, True, "batch_shared", 327, "[1,H,Nq,Nk] over 3 batches, causal"),
    (2, 3, 200, 260, True, "head_shared", 328, "[B,1,Nq,Nk] over 3 heads, causal"),
    (4, 4, 512, 512, True, "alibi", 329, "ALiBi over 4 batches, causal, whole heads per XCD share"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,causal,kind,seed,note", BIAS_CASES)
def test_bwd_bias_full_compare(fa, B, H, Nq, Nk, causal, kind, seed, note):
    import torch
    say(f"case bwd bias={kind} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} seed={seed} ({note})")
    Q, K, V, dO = make_case(B, H, Nq, Nk, seed)
    bias = make_bias(kind, B, H, Nq, Nk, seed + 1)
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    bt = torch.from_numpy(bias).cuda()
    o, lse = fa.fa_fwd(q, k, v, scale=SCALE, causal=causal, bias=bt)
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, g, scale=SCALE, causal=causal, bias=bt)
    torch.cuda.synchronize()
    got = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv)]
    rQ, rK, rV, _, L = oracle.attention_bwd(Q, K, V, dO, SCALE, causal=causal, bias=bias)
    for name, a, b in (("dQ", got[0], rQ), ("dK", got[1], rK), ("dV", got[2], rV)):
        check_grad(name, a, b, note)
    none = np.isneginf(L)
    assert np.all(got[0][none] == 0)


def test_bwd_bias_workload_sampled(fa):
    import torch
    w = fi.WORKLOADS["b2_h16_n8192"]
    say(f"case bwd with a per-key bias [B,H,1,Nk] on {w.name}, causal and not (sampled rows and keys)")
    Q, K, V = fi.make_workload(w)
    dO = fi.make_qkv(w.B, w.H, w.Nq, 1, w.d, seed=w.seed + 5000)[0]
    bias = (2.0 * np.random.default_rng(w.seed + 2).standard_normal((w.B, w.H, 1, w.Nk))).astype(np.float32)
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    bt = torch.from_numpy(bias).cuda()
    rng = np.random.default_rng(w.seed + 3)
    rows = fi.sample_rows(w.B, w.H, w.Nq, 48, seed=w.seed + 4)
    head = int(rng.integers(w.B * w.H))
    keys = np.sort(head * w.Nk + rng.choice(w.Nk, size=16, replace=False)).astype(np.int64)
    keys = np.concatenate([keys, [head * w.Nk, head * w.Nk + w.Nk - 1]]).astype(np.int64)
    for causal in (False, True):
        o, lse = fa.fa_fwd(q, k, v, scale=w.scale, causal=causal, bias=bt)
        dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, g, scale=w.scale, causal=causal, bias=bt)
        torch.cuda.synchronize()
        rQ = oracle.attention_bwd_dq_rows(Q, K, V, dO, w.scale, rows, causal=causal, bias=bias)
        rK, rV = oracle.attention_bwd_dkdv_keys(Q, K, V, dO, w.scale, keys, causal=causal, bias=bias)
        check_grad("dQ rows", dq.float().cpu().numpy().reshape(-1, 128)[rows], rQ, f"bias causal={causal}")
        check_grad("dK keys", dk.float().cpu().numpy().reshape(-1, 128)[keys], rK, f"bias causal={causal}")
        check_grad("dV keys", dv.float().cpu().numpy().reshape(-1, 128)[keys], rV, f"bias causal={causal}")


HD_CASES = [
    # d, d_v, B, H, Nq, Nk, causal, bias kind, seed, note
    (64, 64, 1, 2, 256, 256, False, None, 340, "head size 64, tile aligned"),
    (64, 64, 2, 1, 200, 333, True, None, 341, "head size 64, causal, ragged"),
    (64, 64, 1, 2, 200, 130, False, "per_key_large", 342, "head size 64, per-key bias, ragged"),
    (64, 64, 1, 2, 200, 333, False, "full", 354, "head size 64, dense bias with -inf keys and an empty row"),
    (64, 64, 1, 2, 200, 333, True, "full", 355, "head size 64, dense bias, causal"),
    (64, 64, 2, 2, 300, 300, True, "alibi", 356, "head size 64, ALiBi, causal, several blocks"),
    (192, 128, 1, 2, 256, 256, False, None, 343, "192 / 128, tile aligned"),
    (192, 128, 2, 1, 200, 333, True, None, 344, "192 / 128, causal, ragged"),
    (192, 128, 1, 1, 300, 130, True, None, 345, "192 / 128, causal with Nq > Nk"),
    (192, 128, 1, 2, 200, 333, False, "full", 346, "192 / 128, dense bias with -inf keys and an empty row"),
    (192, 128, 1, 2, 200, 333, True, "full", 347, "192 / 128, dense bias, causal"),
    (192, 128, 1, 2, 1, 700, False, None, 348, "192 / 128, one query row"),
    (256, 256, 1, 2, 256, 256, False, None, 349, "head size 256, tile aligned"),
    (256, 256, 2, 1, 200, 333, True, None, 350, "head size 256, causal, ragged"),
    (256, 256, 1, 1, 300, 130, True, None, 351, "head size 256, causal with Nq > Nk"),
    (256, 256, 1, 2, 200, 333, False, "full", 357, "head size 256, dense bias with -inf keys and an empty row"),
    (256, 256, 1, 2, 200, 333, True, "full", 358, "head size 256, dense bias, causal, ragged"),
    (256, 256, 1, 2, 200, 130, False, "per_key_large", 359, "head size 256, per-key bias with +60 entries"),
    (256, 256, 2, 2, 300, 300, True, "alibi", 360, "head size 256, ALiBi, causal, several blocks"),
    (256, 256, 3, 2, 300, 333, False, "batch_shared", 361, "head size 256, [1,H,Nq,Nk] over 3 batches"),
]


@pytest.mark.parametrize("d,dv,B,H,Nq,Nk,causal,kind,seed,note", HD_CASES)
def test_bwd_head_sizes_full_compare(fa, d, dv, B, H, Nq, Nk, causal, kind, seed, note):
    import torch
    say(f"case bwd d={d} d_v={dv} B={B} H={H} Nq={Nq} Nk={Nk} causal={causal} bias={kind} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, d, seed=seed, dv=dv)
    dO = fi.make_qkv(B, H, Nq, 1, dv, seed=seed + 5000)[0]
    bias = None if kind is None else make_bias(kind, B, H, Nq, Nk, seed + 1)
    sc = 1.0 / math.sqrt(d)
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    bt = None if bias is None else torch.from_numpy(bias).cuda()
    o, lse = fa.fa_fwd(q, k, v, scale=sc, causal=causal, bias=bt)
    dq, dk, dv_, _ = fa.fa_bwd(q, k, v, o, lse, g, scale=sc, causal=causal, bias=bt)
    torch.cuda.synchronize()
    assert tuple(dq.shape) == (B, H, Nq, d) and tuple(dv_.shape) == (B, H, Nk, dv)
    got = [t.float().cpu().numpy().astype(np.float64) for t in (dq, dk, dv_)]
    rQ, rK, rV, _, L = oracle.attention_bwd(Q, K, V, dO, sc, causal=causal, bias=bias)
    for name, a, b in (("dQ", got[0], rQ), ("dK", got[1], rK), ("dV", got[2], rV)):
        check_grad(name, a, b, note)
    assert np.all(got[0][np.isneginf(L)] == 0)


@pytest.mark.parametrize("name", ["b2_h32_n8192_d64", "b2_h16_n8192_d192_dv128", "b2_h8_n8192_d256"])
def test_bwd_head_size_workloads_sampled(fa, name):
    import torch
    w = fi.WORKLOADS[name]
    say(f"case bwd workload {name} (sampled rows and keys)")
    Q, K, V = fi.make_workload(w)
    dO = fi.make_qkv(w.B, w.H, w.Nq, 1, w.d_v, seed=w.seed + 5000)[0]
    q, k, v, g = to_dev(Q), to_dev(K), to_dev(V), to_dev(dO)
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale)
    dq, dk, dv, _ = fa.fa_bwd(q, k, v, o, lse, g, scale=w.scale)
    torch.cuda.synchronize()
    rows = fi.sample_rows(w.B, w.H, w.Nq, 64, seed=w.seed)
    rQ = oracle.attention_bwd_dq_rows(Q, K, V, dO, w.scale, rows)
    rng = np.random.default_rng(w.seed + 1)
    head = int(rng.integers(w.B * w.H))
    keys = np.sort(head * w.Nk + rng.choice(w.Nk, size=16, replace=False)).astype(np.int64)
    keys = np.concatenate([keys, [head * w.Nk, head * w.Nk + w.Nk - 1]]).astype(np.int64)
    rK, rV = oracle.attention_bwd_dkdv_keys(Q, K, V, dO, w.scale, keys)
    check_grad("dQ rows", dq.float().cpu().numpy().reshape(-1, w.d)[rows], rQ, name)
    check_grad("dK keys", dk.float().cpu().numpy().reshape(-1, w.d)[keys], rK, name)
    check_grad("dV keys", dv.float().cpu().numpy().reshape(-1, w.d_v)[keys], rV, name)
