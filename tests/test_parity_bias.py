"""GPU parity of the mask/bias term with an fp32 additive bias (alone and
with the causal mask) against the fp64 oracle, element by element.

The bias enters the score equation of "FlashAttention'ı Anlamak Bölüm 1",
section 0.2, as an additive term; the oracle adds it in fp64 to the scaled
dot product.  Bias layouts cover the broadcast forms a caller passes
(per element, per head and key, per row and key, ALiBi-like distance
penalties), ragged lengths, keys hidden with -inf, rows that see no key, and
large offsets that move the running max late in the key loop.
"""
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


def alibi(H, Nq, Nk):
    """-2^-(h+1) * |i + (Nk - Nq) - j| in float32 (exact: power-of-two slopes)."""
    i = np.arange(Nq, dtype=np.int64)[:, None] + (Nk - Nq)
    j = np.arange(Nk, dtype=np.int64)[None, :]
    dist = np.abs(i - j).astype(np.float32)
    slopes = np.float32(2.0) ** -(np.arange(H, dtype=np.float32) + 1)
    return (-slopes[:, None, None] * dist[None]).astype(np.float32)[None]  # [1, H, Nq, Nk]


def make_bias(kind, B, H, Nq, Nk, seed):
    rng = np.random.default_rng(seed + 7777)
    if kind == "full":
        return (2.0 * rng.standard_normal((B, H, Nq, Nk))).astype(np.float32)
    if kind == "per_head_key":
        return (2.0 * rng.standard_normal((1, H, 1, Nk))).astype(np.float32)
    if kind == "rows_keys":
        return (2.0 * rng.standard_normal((Nq, Nk))).astype(np.float32)
    if kind == "alibi":
        return alibi(H, Nq, Nk)
    if kind == "batch_shared":
        return (2.0 * rng.standard_normal((1, H, Nq, Nk))).astype(np.float32)
    if kind == "head_shared":
        return (2.0 * rng.standard_normal((B, 1, Nq, Nk))).astype(np.float32)
    raise ValueError(kind)


def run(fa, Q, K, V, bias, causal=False, scale=SCALE):
    import torch
    bt = torch.from_numpy(np.ascontiguousarray(bias)).cuda()
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=scale, causal=causal, bias=bt)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


def compare_all(Og, Lg, Oo, Lo, label):
    none = np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), none), "rows that see no key must report LSE = -inf"
    assert np.all(Og[none] == 0)
    check_parity(Og[~none], Lg[~none], Oo[~none], Lo[~none], label)


BIAS_CASES = [
    # B, H, Nq, Nk, bias layout, causal, seed, note
    (1, 2, 256, 256, "full", False, 90, "full [B,H,Nq,Nk], tile aligned"),
    (2, 3, 200, 333, "full", False, 91, "ragged Nq and Nk"),
    (1, 2, 130, 97, "per_head_key", False, 92, "[1,H,1,Nk], Nk % 4 = 1 (padded copy)"),
    (2, 1, 300, 260, "rows_keys", True, 93, "[Nq,Nk] over batch and heads, causal"),
    (1, 1, 129, 65, "full", True, 94, "causal, one row past a q tile, one key past a kv tile"),
    (1, 2, 64, 1, "full", False, 95, "single key"),
    (1, 2, 640, 640, "alibi", False, 96, "ALiBi-like slopes, several q tiles"),
    (1, 1, 300, 130, "full", True, 97, "causal with Nq > Nk: leading rows see no key"),
    # bias rows shared by several heads: their workgroups are grouped in the grid
    (3, 2, 300, 333, "batch_shared", False, 102, "[1,H,Nq,Nk] over 3 batches, ragged"),
    (3, 2, 300, 333, "batch_shared", True, 103, "[1,H,Nq,Nk] over 3 batches, causal"),
    (2, 3, 200, 260, "head_shared", False, 104, "[B,1,Nq,Nk] over 3 heads"),
    (2, 3, 200, 260, "head_shared", True, 105, "[B,1,Nq,Nk] over 3 heads, causal"),
    (2, 3, 257, 190, "rows_keys", False, 106, "[Nq,Nk] over 2 batches and 3 heads"),
    (4, 4, 512, 256, "batch_shared", True, 107, "[1,H,Nq,Nk], whole heads per XCD share (64 workgroups)"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,kind,causal,seed,note", BIAS_CASES)
def test_bias_full_compare(fa, B, H, Nq, Nk, kind, causal, seed, note):
    say(f"case bias {kind} causal={causal} B={B} H={H} Nq={Nq} Nk={Nk} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed)
    bias = make_bias(kind, B, H, Nq, Nk, seed)
    Og, Lg = run(fa, Q, K, V, bias, causal)
    Oo, Lo = oracle.attention_masked(Q, K, V, SCALE, causal=causal, bias=bias)
    compare_all(Og, Lg, Oo, Lo, f"bias {note}")


def test_bias_negative_scale(fa):
    say("case bias with a negative scale")
    Q, K, V = fi.make_qkv(1, 2, 200, 170, 128, seed=98)
    bias = make_bias("full", 1, 2, 200, 170, 98)
    Og, Lg = run(fa, Q, K, V, bias, scale=-0.3)
    Oo, Lo = oracle.attention_masked(Q, K, V, -0.3, bias=bias)
    compare_all(Og, Lg, Oo, Lo, "bias, scale -0.3")


def test_bias_minus_inf_hides_keys(fa):
    say("case -inf bias entries: hidden keys and a row that sees none")
    B, H, Nq, Nk = 1, 2, 150, 210
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=99)
    rng = np.random.default_rng(99)
    bias = rng.standard_normal((B, H, Nq, Nk)).astype(np.float32)
    bias[rng.random(bias.shape) < 0.3] = -np.inf
    bias[0, 0, 17, :] = -np.inf          # row 17 of head 0 sees no key
    bias[0, 1, 5, :-1] = -np.inf         # row 5 of head 1 sees only the last key
    Og, Lg = run(fa, Q, K, V, bias)
    Oo, Lo = oracle.attention_masked(Q, K, V, SCALE, bias=bias)
    assert np.isneginf(Lo[0, 0, 17])
    compare_all(Og, Lg, Oo, Lo, "bias with -inf entries")


def test_bias_late_max_jump(fa):
    say("case large bias on late keys: the running max rises in the last tiles")
    B, H, Nq, Nk = 1, 2, 256, 1000
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=100)
    bias = np.zeros((1, H, 1, Nk), np.float32)
    bias[..., 700:] = 12.0
    bias[..., 990:] = 40.0
    Og, Lg = run(fa, Q, K, V, bias)
    Oo, Lo = oracle.attention_masked(Q, K, V, SCALE, bias=bias)
    compare_all(Og, Lg, Oo, Lo, "bias max jump")


def test_bias_alibi_sampled(fa):
    import torch
    B, H, N = 1, 4, 4096
    say(f"case ALiBi bias sampled B={B} H={H} N={N}, causal and not")
    Q, K, V = fi.make_qkv(B, H, N, N, 128, seed=101, k_scale=4.0, offset_frac=0.01, offset=8.0)
    bias = alibi(H, N, N)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    bt = torch.from_numpy(bias).cuda()
    rows = fi.sample_rows(B, H, N, 128, seed=101)
    idx = torch.from_numpy(rows).cuda()
    for causal in (False, True):
        o, lse = fa.fa_fwd(q, k, v, scale=SCALE, causal=causal, bias=bt)
        torch.cuda.synchronize()
        Or, Lr = oracle.attention_masked(Q, K, V, SCALE, causal=causal, bias=bias, rows=rows)
        check_parity(o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64),
                     lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr,
                     f"alibi sampled causal={causal}")


def test_bias_deterministic_and_strided(fa):
    import torch
    say("case bias: repeat calls bit-identical; a strided view equals its copy")
    Q, K, V = fi.make_qkv(2, 2, 190, 260, 128, seed=102)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    big = torch.randn(2, 2, 190, 300, device="cuda")
    view = big[..., 20:280]                 # row stride 300, base offset 80 bytes
    o1, l1 = fa.fa_fwd(q, k, v, bias=view)
    o2, l2 = fa.fa_fwd(q, k, v, bias=view.contiguous())
    o3, l3 = fa.fa_fwd(q, k, v, bias=view)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o3.view(torch.int16)) and torch.equal(l1, l3)
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
