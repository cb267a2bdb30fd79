"""GPU parity of fa_fwd (through the C ABI) against the fp64 CPU oracle.

Small and ragged shapes and the five full-size workloads (in the launch
configuration the benchmark times) are compared element by element over the
whole output.
"""
import math
import time

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


def run_gpu(fa, Q, K, V, scale):
    import torch
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=scale)
    torch.cuda.synchronize()
    return o_to_f64(o), lse.cpu().numpy().astype(np.float64)


SMALL = [
    # B, H, Nq, Nk, seed, note
    (1, 1, 256, 256, 1001, "tiny workload shape"),
    (1, 1, 128, 64, 31, "one q tile, one kv tile"),
    (2, 3, 200, 300, 32, "ragged q and kv tails"),
    (1, 2, 1, 1, 33, "single query, single key"),
    (1, 1, 77, 1000, 34, "short q, ragged long kv"),
    (2, 2, 129, 65, 35, "one row past a q tile, one key past a kv tile"),
    (1, 1, 640, 129, 36, "several q tiles"),
    (3, 1, 33, 7, 37, "kv shorter than a tile"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,seed,note", SMALL)
def test_small_and_ragged_full_compare(fa, B, H, Nq, Nk, seed, note):
    say(f"case small B={B} H={H} Nq={Nq} Nk={Nk} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed)
    sc = 1.0 / math.sqrt(128)
    Og, Lg = run_gpu(fa, Q, K, V, sc)
    Oo, Lo = oracle.attention(Q, K, V, sc)
    check_parity(Og, Lg, Oo, Lo, note)


@pytest.mark.parametrize("scale,note", [(0.0, "zero scale"), (-0.0883883476, "negative scale"),
                                        (0.5, "large scale"), (4.0, "near-hardmax scale")])
def test_scale_variants(fa, scale, note):
    say(f"case scale={scale} ({note})")
    Q, K, V = fi.make_qkv(1, 2, 192, 320, 128, seed=40)
    Og, Lg = run_gpu(fa, Q, K, V, scale)
    Oo, Lo = oracle.attention(Q, K, V, scale)
    check_parity(Og, Lg, Oo, Lo, note)


@pytest.mark.parametrize("causal", [False, True])
def test_zero_scale_with_masked_tiles(fa, causal):
    # hidden keys carry -inf scores; with scale 0 they must still weigh 0
    import torch
    say(f"case zero scale, ragged keys, causal={causal}")
    Q, K, V = fi.make_qkv(1, 2, 190, 260, 128, seed=41)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=0.0, causal=causal)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attention_masked(Q, K, V, 0.0, causal=causal)
    check_parity(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Oo, Lo, f"zero scale causal={causal}")


def test_large_logits_and_max_jumps(fa):
    # same value recipe as the 16K workload, at a size the oracle finishes in seconds
    say("case koffset small: K*4, 1% rows +8, B=1 H=2 Nq=256 Nk=2048")
    Q, K, V = fi.make_qkv(1, 2, 256, 2048, 128, seed=41, k_scale=4.0, offset_frac=0.01, offset=8.0)
    sc = 1.0 / math.sqrt(128)
    Og, Lg = run_gpu(fa, Q, K, V, sc)
    Oo, Lo = oracle.attention(Q, K, V, sc)
    check_parity(Og, Lg, Oo, Lo, "koffset small")


def test_identical_keys_give_mean_of_v(fa):
    say("case identical keys")
    Q, K, V = fi.make_qkv(1, 1, 128, 512, 128, seed=42)
    K[:] = K[:, :, :1, :]
    Og, Lg = run_gpu(fa, Q, K, V, 1 / math.sqrt(128))
    mean_v = fi.bf16_bits_to_f32(V).astype(np.float64).mean(axis=2, keepdims=True)
    assert np.abs(Og - mean_v).max() < 4e-3
    q = fi.bf16_bits_to_f32(Q).astype(np.float64)[0, 0]
    k = fi.bf16_bits_to_f32(K).astype(np.float64)[0, 0, 0]
    expect = np.float64(np.float32(1 / math.sqrt(128))) * (q @ k) + math.log(512)
    assert np.abs(Lg[0, 0] - expect).max() < 1e-3


def test_constant_v_column_and_permutation(fa):
    say("case constant V column + key permutation")
    Q, K, V = fi.make_qkv(1, 2, 256, 384, 128, seed=43)
    V[..., 17] = fi.f32_to_bf16_bits(np.float32(2.5))
    Og, Lg = run_gpu(fa, Q, K, V, 1 / math.sqrt(128))
    assert np.abs(Og[..., 17] - 2.5).max() <= 2 ** -7  # one bf16 ulp at 2.5
    perm = np.random.default_rng(44).permutation(384)
    Og2, Lg2 = run_gpu(fa, Q, np.ascontiguousarray(K[:, :, perm]), np.ascontiguousarray(V[:, :, perm]),
                       1 / math.sqrt(128))
    assert np.abs(Og2 - Og).max() < 4e-3 and np.abs(Lg2 - Lg).max() < 1e-4


def test_empty_query_is_noop(fa):
    import torch
    q = torch.zeros(1, 2, 0, 128, dtype=torch.bfloat16, device="cuda")
    k = torch.zeros(1, 2, 5, 128, dtype=torch.bfloat16, device="cuda")
    o, lse = fa.fa_fwd(q, k, k)
    torch.cuda.synchronize()
    assert o.shape == (1, 2, 0, 128) and lse.shape == (1, 2, 0)


def test_deterministic(fa):
    import torch
    say("case determinism")
    Q, K, V = fi.make_qkv(2, 2, 384, 1000, 128, seed=45)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o1, l1 = fa.fa_fwd(q, k, v)
    o2, l2 = fa.fa_fwd(q, k, v)
    torch.cuda.synchronize()
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)


@pytest.mark.parametrize("name", fi.WORKLOAD_ORDER)
def test_workloads_full_compare(fa, name):
    """Every output element of each workload, at its full size and in the
    launch configuration the benchmark times, against the whole fp64 oracle
    (the 5090 benchmark row of "Flash Attention на 5090 в CUDA C++" and the
    4K/8K/16K lengths of the B200 article's lead)."""
    import time

    import torch
    w = fi.WORKLOADS[name]
    say(f"case workload {name}: {w.describe()} (full compare)")
    Q, K, V = fi.make_workload(w)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o, lse = fa.fa_fwd(q, k, v, scale=w.scale)
    torch.cuda.synchronize()
    Og, Lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    del q, k, v, o, lse
    t0 = time.perf_counter()
    Oo, Lo = oracle.attention(Q, K, V, w.scale)
    say(f"  oracle: {w.B * w.H * w.Nq} rows in {time.perf_counter() - t0:.1f} s "
        f"on {oracle.max_threads()} threads")
    check_parity(Og, Lg, Oo, Lo, f"{name} (all {Og.size} elements)")


def test_single_hip_runtime(fa):
    # torch and libfa06.so must share one HIP runtime, or torch's stream
    # handles would be meaningless to the library.
    maps = open("/proc/self/maps").read().splitlines()
    paths = {ln.split()[-1] for ln in maps if "libamdhip64" in ln}
    assert len(paths) == 1, paths
    assert any("libfa06.so" in ln for ln in maps)


# Shapes whose grid holds at least 256 workgroups of 256 query rows
# (B*H*ceil(Nq/256) >= 256): these run the 8-wave head-size-128 kernel with
# the segmented iteration.
SEG_CASES = [
    # B, H, Nq, Nk, seed, scale, kwargs, note
    (1, 256, 300, 200, 50, None, {}, "ragged q tile (44 rows) and kv tail (8 keys)"),
    (2, 128, 256, 1000, 51, None, {}, "seven segmented iteration pairs, ragged kv"),
    (1, 256, 1, 64, 52, None, {}, "one query row per head, one kv tile"),
    (1, 256, 256, 640, 53, -0.0883883476, {}, "negative scale"),
    (1, 256, 256, 1024, 54, None, dict(k_scale=4.0, offset_frac=0.01, offset=8.0),
     "large logits, running-max jumps (the 16K workload's recipe)"),
]


# Shapes whose grid holds fewer than 256 workgroups of 256 rows but at least
# 256 of 128 rows, with at least 1024 keys: the 8-wave kernel with two key
# groups per workgroup (each attends to half of the key tiles, then the two
# halves are merged in LDS).
KS2_CASES = [
    # B, H, Nq, Nk, seed, scale, kwargs, note
    (1, 128, 256, 1024, 60, None, {}, "16 tiles, 8 per key group"),
    (1, 128, 200, 1087, 61, None, {}, "17 tiles: ragged 17th, the second group's 9th tile past the keys"),
    (2, 64, 256, 1100, 62, None, {}, "18 tiles, ragged last"),
    (1, 128, 256, 2000, 63, -0.07, dict(k_scale=4.0, offset_frac=0.01, offset=8.0),
     "negative scale, large logits (the 16K workload's recipe)"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,seed,scale,kw,note", KS2_CASES)
def test_key_group_kernel_full_compare(fa, B, H, Nq, Nk, seed, scale, kw, note):
    assert B * H * ((Nq + 255) // 256) < 256 <= B * H * ((Nq + 127) // 128) <= 512 and Nk >= 1024
    say(f"case 8-wave key groups B={B} H={H} Nq={Nq} Nk={Nk} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed, **kw)
    sc = 1.0 / math.sqrt(128) if scale is None else scale
    Og, Lg = run_gpu(fa, Q, K, V, sc)
    Oo, Lo = oracle.attention(Q, K, V, sc)
    check_parity(Og, Lg, Oo, Lo, f"8-wave key groups {note}")


@pytest.mark.parametrize("B,H,Nq,Nk,seed,scale,kw,note", SEG_CASES)
def test_eight_wave_kernel_full_compare(fa, B, H, Nq, Nk, seed, scale, kw, note):
    say(f"case 8-wave B={B} H={H} Nq={Nq} Nk={Nk} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed, **kw)
    sc = 1.0 / math.sqrt(128) if scale is None else scale
    Og, Lg = run_gpu(fa, Q, K, V, sc)
    Oo, Lo = oracle.attention(Q, K, V, sc)
    check_parity(Og, Lg, Oo, Lo, f"8-wave {note}")


CAUSAL_CASES = [
    # B, H, Nq, Nk, seed, note
    (1, 2, 256, 256, 80, "square, tile aligned"),
    (2, 1, 200, 333, 81, "Nk > Nq, ragged"),
    (1, 2, 300, 130, 82, "Nq > Nk: leading rows see no key"),
    (1, 1, 1, 1, 83, "single query and key"),
    (1, 1, 129, 65, 84, "one row past a q tile, one key past a kv tile"),
    (1, 1, 640, 640, 85, "several q tiles, diagonal through every one"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,seed,note", CAUSAL_CASES)
def test_causal_full_compare(fa, B, H, Nq, Nk, seed, note):
    import torch
    say(f"case causal B={B} H={H} Nq={Nq} Nk={Nk} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=1 / math.sqrt(128), causal=True)
    torch.cuda.synchronize()
    Og, Lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    Oo, Lo = oracle.attention_masked(Q, K, V, 1 / math.sqrt(128), causal=True)
    none = np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), none), "rows that see no key must report LSE = -inf"
    assert np.all(Og[none] == 0)
    check_parity(Og[~none], Lg[~none], Oo[~none], Lo[~none], f"causal {note}")


# Causal launches of the same size class run the key groups too: each group
# takes half of the tiles its q-tile sees, the second half holding the
# diagonal; rows that see none of a group's keys get weight 0 in the merge.
KS2_CAUSAL_CASES = [
    # B, H, Nq, Nk, seed, note
    (1, 128, 256, 1024, 86, "Nk > Nq: every row sees 768 keys and more"),
    (1, 128, 200, 1087, 87, "ragged q and kv tails"),
    (1, 32, 1280, 1024, 88, "Nq > Nk: the first 256 rows see no key, whole q-tiles empty"),
    (2, 64, 256, 1100, 89, "two batches"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,seed,note", KS2_CAUSAL_CASES)
def test_causal_key_group_kernel_full_compare(fa, B, H, Nq, Nk, seed, note):
    import torch
    assert B * H * ((Nq + 255) // 256) < 256 <= B * H * ((Nq + 127) // 128) <= 512 and Nk >= 1024
    say(f"case causal 8-wave key groups B={B} H={H} Nq={Nq} Nk={Nk} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=1 / math.sqrt(128), causal=True)
    torch.cuda.synchronize()
    Og, Lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    Oo, Lo = oracle.attention_masked(Q, K, V, 1 / math.sqrt(128), causal=True)
    none = np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), none), "rows that see no key must report LSE = -inf"
    assert np.all(Og[none] == 0)
    check_parity(Og[~none], Lg[~none], Oo[~none], Lo[~none], f"causal key groups {note}")


def test_causal_offset_keys_sampled(fa):
    import torch
    say("case causal koffset: K*4, 1% rows +8, B=1 H=4 N=4096")
    Q, K, V = fi.make_qkv(1, 4, 4096, 4096, 128, seed=86, k_scale=4.0, offset_frac=0.01, offset=8.0)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=1 / math.sqrt(128), causal=True)
    torch.cuda.synchronize()
    rows = fi.sample_rows(1, 4, 4096, 192, seed=86)
    Or, Lr = oracle.attention_masked(Q, K, V, 1 / math.sqrt(128), causal=True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check_parity(o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64),
                 lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr, "causal koffset (sampled)")


# Causal launches of at least 8192 query rows on grids of >= 256 workgroups
# of 256 rows run the 8-wave kernel (segmented plain tiles, masked diagonal).
EIGHT_WAVE_CAUSAL_CASES = [
    # B, H, Nq, Nk, seed, note
    (1, 8, 8192, 8192, 90, "square: 32 diagonal tiles of 256 rows per head"),
    (1, 8, 8492, 8000, 91, "Nq > Nk: 492 leading rows see no key, ragged q tile and kv tail"),
]


@pytest.mark.parametrize("B,H,Nq,Nk,seed,note", EIGHT_WAVE_CAUSAL_CASES)
def test_causal_eight_wave_full_compare(fa, B, H, Nq, Nk, seed, note):
    import torch
    say(f"case causal 8-wave B={B} H={H} Nq={Nq} Nk={Nk} seed={seed} ({note})")
    Q, K, V = fi.make_qkv(B, H, Nq, Nk, 128, seed=seed)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=1 / math.sqrt(128), causal=True)
    torch.cuda.synchronize()
    Og, Lg = o_to_f64(o), lse.cpu().numpy().astype(np.float64)
    t0 = time.time()
    Oo, Lo = oracle.attention_masked(Q, K, V, 1 / math.sqrt(128), causal=True)
    say(f"  oracle: {B * H * Nq} rows in {time.time() - t0:.1f} s")
    none = np.isneginf(Lo)
    assert np.array_equal(np.isneginf(Lg), none), "rows that see no key must report LSE = -inf"
    assert np.all(Og[none] == 0)
    check_parity(Og[~none], Lg[~none], Oo[~none], Lo[~none], f"causal 8-wave {note}")


@pytest.mark.parametrize("scale,note", [(-1 / math.sqrt(128), "negative scale"), (0.0, "zero scale")])
def test_causal_eight_wave_scales(fa, scale, note):
    import torch
    say(f"case causal 8-wave B=1 H=8 N=8192 scale={scale} ({note})")
    Q, K, V = fi.make_qkv(1, 8, 8192, 8192, 128, seed=92)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=scale, causal=True)
    torch.cuda.synchronize()
    Oo, Lo = oracle.attention_masked(Q, K, V, scale, causal=True)
    check_parity(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Oo, Lo, f"causal 8-wave {note}")


@pytest.mark.parametrize("scale,note", [(-1 / math.sqrt(128), "negative scale"), (0.0, "zero scale")])
def test_key_group_kernel_scales(fa, scale, note):
    import torch
    say(f"case 8-wave key groups B=1 H=128 Nq=256 Nk=1100 scale={scale} ({note}), causal and not")
    Q, K, V = fi.make_qkv(1, 128, 256, 1100, 128, seed=93)
    for causal in (False, True):
        o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=scale, causal=causal)
        torch.cuda.synchronize()
        Oo, Lo = oracle.attention_masked(Q, K, V, scale, causal=causal)
        check_parity(o_to_f64(o), lse.cpu().numpy().astype(np.float64), Oo, Lo,
                     f"key groups {note} causal={causal}")


def test_causal_eight_wave_offset_keys_sampled(fa):
    import torch
    w = fi.WORKLOADS["b1_h16_n16384_koffset"]
    say("case causal 8-wave on the 16K offset-key workload (sampled rows)")
    Q, K, V = fi.make_workload(w)
    o, lse = fa.fa_fwd(to_dev(Q), to_dev(K), to_dev(V), scale=w.scale, causal=True)
    torch.cuda.synchronize()
    rows = fi.sample_rows(w.B, w.H, w.Nq, 256, seed=w.seed)
    Or, Lr = oracle.attention_masked(Q, K, V, w.scale, causal=True, rows=rows)
    idx = torch.from_numpy(rows).cuda()
    check_parity(o.view(-1, 128)[idx].float().cpu().numpy().astype(np.float64),
                 lse.view(-1)[idx].cpu().numpy().astype(np.float64), Or, Lr, "causal 8-wave koffset (sampled)")


def test_noncausal_unchanged_by_masked_entry(fa):
    import torch
    Q, K, V = fi.make_qkv(1, 2, 200, 300, 128, seed=87)
    q, k, v = to_dev(Q), to_dev(K), to_dev(V)
    o1, l1 = fa.fa_fwd(q, k, v)
    o2 = torch.empty_like(o1)
    l2 = torch.empty_like(l1)
    rc = fa.fa_fwd_masked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o2.data_ptr(), l2.data_ptr(),
                              1, 2, 200, 300, 128, 1 / math.sqrt(128), 0, None, 0, 0, 0,
                              torch.cuda.current_stream().cuda_stream)
    torch.cuda.synchronize()
    assert rc == 0
    assert torch.equal(o1.view(torch.int16), o2.view(torch.int16)) and torch.equal(l1, l2)
