"""The C-ABI library on the CPU: it loads, exports what include/fa06.h
declares, and rejects bad arguments before any HIP call (so no GPU is needed)."""
import ctypes
import os
import re

import pytest

import flashattention_forward_06_amd as fa

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "fa06.h")


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(fa_[a-z0-9_]+)\s*\(", text)))


def test_library_exports_every_declared_function():
    lib = fa.load_library()
    names = declared_functions()
    assert names == ["fa_build_info", "fa_bwd", "fa_bwd_build_info", "fa_bwd_dv", "fa_bwd_masked", "fa_fwd",
                     "fa_fwd_dv",
                     "fa_fwd_masked",
                     "fa_fwd_mxfp8", "fa_fwd_splitkv", "fa_fwd_splitkv_noalloc", "fa_fwd_splitkv_noalloc_max_bytes",
                     "fa_fwd_splitkv_workspace_bytes",
                     "fa_mxfp8_build_info", "fa_mxfp8_quantize_rows", "fa_mxfp8_quantize_vt", "fa_status_string"]
    for n in names:
        assert hasattr(lib, n), f"{n} declared in fa06.h but not exported"


def test_status_strings():
    for code, name in fa.STATUS.items():
        assert fa.fa_status_string(code).startswith(name)
    assert "unknown" in fa.fa_status_string(99)
    assert "gfx950" in fa.fa_build_info()


# Fake, well-aligned addresses: never dereferenced, because every call below
# fails validation before the library touches HIP.
Qp, Kp, Vp = 0x10000000, 0x20000000, 0x30000000
Op, Lp = 0x40000000, 0x50000000
GOOD = dict(B=1, H=2, Nq=256, Nk=256, d=128, scale=0.088)


def call(q=Qp, k=Kp, v=Vp, o=Op, lse=Lp, **kw):
    a = {**GOOD, **kw}
    return fa.fa_fwd_raw(q, k, v, o, lse, a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(k=0), 1), (dict(v=0), 1), (dict(o=0), 1), (dict(lse=0), 1),
    (dict(B=-1), 2), (dict(H=-1), 2), (dict(Nq=-1), 2), (dict(Nk=0), 2), (dict(Nk=-5), 2),
    (dict(B=1 << 40, H=1 << 40), 2),
    (dict(d=32), 3), (dict(d=96), 3), (dict(d=512), 3), (dict(Nq=(1 << 23) + 1), 3), (dict(Nk=(1 << 23) + 1), 3),
    (dict(d=256, Nk=(1 << 22) + 1), 3), (dict(d=256, Nq=(1 << 22) + 1), 3),   # 2^31-byte head slices
    (dict(q=Qp + 8), 3), (dict(k=Kp + 2), 3), (dict(v=Vp + 4), 3), (dict(o=Op + 8), 3), (dict(lse=Lp + 2), 3),
    (dict(o=Qp), 4), (dict(o=Kp + 256), 4), (dict(lse=Vp + 1024), 4), (dict(lse=Op + 4096), 4),
    (dict(scale=float("nan")), 5), (dict(scale=float("inf")), 5), (dict(scale=float("-inf")), 5),
])
def test_validation_codes(kw, code):
    assert call(**kw) == code


def call_masked(causal=1, bias=None, sb=0, sh=0, sq=0, **kw):
    a = {**GOOD, **kw}
    return fa.fa_fwd_masked_raw(Qp, Kp, Vp, Op, Lp, a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"],
                                causal, bias, sb, sh, sq, 0)


BIAS_P = 0x60000000  # a 16-byte aligned address clear of the other fake buffers


def test_masked_entry_validation():
    assert call_masked(causal=2) == 3
    assert call_masked(causal=-1) == 3
    assert call_masked(Nk=0) == 2
    assert call_masked(d=96) == 3
    assert call_masked(scale=float("nan")) == 5
    assert call_masked(Nq=0) == 0
    assert call_masked(Nq=0, bias=BIAS_P) == 0          # empty problem: no-op


@pytest.mark.parametrize("kw,code", [
    (dict(bias=BIAS_P + 4), 3),                         # base not 16-byte aligned
    (dict(bias=BIAS_P, sq=258), 3),                     # row stride not a multiple of 4
    (dict(bias=BIAS_P, sh=6, sq=256), 3),
    (dict(bias=BIAS_P, sb=2, sq=256), 3),
    (dict(bias=BIAS_P, sq=-256), 3),                    # negative strides
    (dict(bias=BIAS_P, sh=-4), 3),
    (dict(bias=BIAS_P, sq=1 << 25), 3),                 # 32 rows span more than 2^29 elements
    (dict(bias=BIAS_P, sb=1 << 62, B=3), 2),            # extent beyond 2^60 elements
    (dict(bias=Op - 4096, sq=256), 4),                  # bias rows overlap O
    (dict(bias=Lp, sq=0), 4),                           # bias overlaps LSE
    (dict(bias=Qp, sq=256), -1),                        # reading Q as bias is allowed
    (dict(bias=BIAS_P, sq=256, sh=256 * 256), -1),      # valid: fails only at the device check
    (dict(bias=BIAS_P, causal=0), -1),                  # broadcast over everything, no causal mask
])
def test_bias_validation(kw, code):
    if code == -1:
        # arguments accepted: without a GPU the call stops at the device
        # check; with one it would launch on these fake addresses, so skip
        import torch
        if torch.cuda.is_available():
            pytest.skip("would launch on fake pointers")
        assert call_masked(**kw) == 6
    else:
        assert call_masked(**kw) == code


def test_empty_problem_is_noop():
    # B*H*Nq == 0 returns success without touching the device
    assert call(Nq=0) == 0
    assert call(B=0) == 0
    assert call(H=0) == 0
    # empty buffers may come with NULL pointers (torch's empty tensors do)
    assert call(Nq=0, q=0, o=0, lse=0) == 0
    assert call(B=0, q=0, k=0, v=0, o=0, lse=0) == 0
    # but K and V are not empty when Nq == 0
    assert call(Nq=0, k=0) == 1


def test_no_device_reports_device_error():
    import torch
    if torch.cuda.is_available():
        pytest.skip("a GPU is present; this case is for hosts without one")
    assert call() == 6


def test_python_wrapper_type_checks():
    import torch
    x = torch.zeros(1, 1, 4, 128, dtype=torch.bfloat16)
    with pytest.raises(TypeError):
        fa.fa_fwd(x.float(), x, x)
    with pytest.raises(ValueError):
        fa.fa_fwd(x[0], x, x)
    with pytest.raises(ValueError):
        fa.fa_fwd(x, x, x)  # CPU tensors are rejected


def test_missing_library_fails_loudly(tmp_path):
    with pytest.raises(ImportError):
        fa.load_library(str(tmp_path / "nope.so"))


# backward: fake buffers for O, dO, dQ, dK, dV and D
Op2, dOp = 0x70000000, 0x80000000
dQp, dKp, dVp, Dp = 0x90000000, 0xA0000000, 0xB0000000, 0xC0000000
GOOD_BWD = dict(q=Qp, k=Kp, v=Vp, o=Op2, do=dOp, lse=Lp, dq=dQp, dk=dKp, dv=dVp, dl=Dp,
                B=1, H=2, Nq=256, Nk=256, d=128, scale=0.088, causal=0)


def call_bwd(**kw):
    a = {**GOOD_BWD, **kw}
    return fa.fa_bwd_raw(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["dl"],
                         a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], 0)


@pytest.mark.parametrize("kw,code", [
    (dict(q=0), 1), (dict(do=0), 1), (dict(lse=0), 1), (dict(dq=0), 1), (dict(dk=0), 1), (dict(dl=0), 1),
    (dict(B=-1), 2), (dict(Nk=0), 2), (dict(Nq=-3), 2),
    (dict(d=96), 3), (dict(d=32), 3), (dict(d=192), 3), (dict(causal=2), 3), (dict(Nk=(1 << 23) + 1), 3),
    (dict(o=Op2 + 8), 3), (dict(dv=dVp + 4), 3), (dict(dl=Dp + 2), 3),
    (dict(dq=Qp), 4), (dict(dk=Kp + 256), 4), (dict(dv=dKp), 4), (dict(dl=Lp), 4), (dict(dq=dOp + 512), 4),
    (dict(scale=float("nan")), 5),
    (dict(B=0), 0),
])
def test_bwd_validation_codes(kw, code):
    assert call_bwd(**kw) == code


BIASp = 0x60000000  # a free slot among the fake buffers


def call_bwd_bias(bias=BIASp, sb=0, sh=0, sq=256, **kw):
    a = {**GOOD_BWD, **kw}
    return fa.fa_bwd_masked_raw(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"],
                                a["dl"], a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["scale"], a["causal"], bias,
                                sb, sh, sq, 0)


@pytest.mark.parametrize("kw,code", [
    (dict(sq=-4), 3), (dict(sh=6), 3), (dict(bias=BIASp + 4), 3),
    (dict(sq=1 << 28), 3),                          # (Nq-1)*sq + Nk beyond 2^29: a key column's span
    (dict(sb=1 << 58, B=8), 2),                     # extent beyond 2^60 elements
    (dict(bias=dKp), 4), (dict(bias=Dp - 64), 4),   # overlaps dK / D
    (dict(bias=Qp), None), (dict(bias=0), None),    # may alias an input; NULL is plain fa_bwd
])
def test_bwd_bias_validation_codes(kw, code):
    import torch
    if code is None:
        if torch.cuda.is_available():
            pytest.skip("would launch on fake pointers")
        code = 6
    assert call_bwd_bias(**kw) == code


def call_bwd_dv(hd=192, hdv=128, **kw):
    """fa_bwd_dv on the fake buffers; hd, hdv are the head sizes (kw keys
    override GOOD_BWD's pointers and sizes)."""
    a = {**GOOD_BWD, **kw}
    return fa.fa_bwd_dv_raw(a["q"], a["k"], a["v"], a["o"], a["do"], a["lse"], a["dq"], a["dk"], a["dv"], a["dl"],
                            a["B"], a["H"], a["Nq"], a["Nk"], hd, hdv, a["scale"], a["causal"], None, 0, 0, 0, 0)


# extents at B=1, H=2, Nq=Nk=256: Q, K, dQ, dK (d=192) 196608 bytes; V, O, dO, dV (d_v=128) 131072
@pytest.mark.parametrize("kw,code", [
    (dict(hd=192, hdv=192), 3), (dict(hd=128, hdv=64), 3), (dict(hd=256, hdv=128), 3), (dict(hd=512, hdv=512), 3),
    (dict(Nk=(1 << 30) // 192 + 1), 3),
    (dict(dq=Kp + 131072), 4),        # inside K only because K rows are 192 wide
    (dict(dl=dOp + 131068), 4),       # last dword of dO (d_v wide)
    (dict(Nk=0), 2), (dict(o=0), 1),
])
def test_bwd_dv_validation_codes(kw, code):
    assert call_bwd_dv(**kw) == code


def test_bwd_other_head_sizes_reach_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch on fake pointers")
    assert call_bwd(d=64) == 6
    assert call_bwd_dv(hd=64, hdv=64) == 6 and call_bwd_dv(hd=128, hdv=128) == 6 and call_bwd_dv() == 6
    assert call_bwd_dv(dq=Kp + 196608) == 6   # just past K's 192-wide extent: no alias


def test_bwd_accepted_arguments_reach_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch on fake pointers")
    assert call_bwd() == 6
    assert call_bwd(Nq=0) == 6     # dK and dV must still be zeroed on the device


def test_other_head_sizes_reach_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch on fake pointers")
    for d in (64, 128, 256):
        assert call(d=d) == 6


# fa_fwd_dv: value head size d_v apart from the query/key head size d
def call_dv(q=Qp, k=Kp, v=Vp, o=Op, lse=Lp, **kw):
    a = {**GOOD, "d": 192, "dv": 128, "causal": 0, **kw}
    return fa.fa_fwd_dv_raw(q, k, v, o, lse, a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["dv"], a["scale"],
                            a["causal"], None, 0, 0, 0, 0)


# extents at B=1, H=2, Nq=Nk=256: K (d=192) 196608 bytes, V and O (d_v=128) 131072
@pytest.mark.parametrize("kw,code", [
    (dict(d=192, dv=192), 3), (dict(d=128, dv=64), 3), (dict(d=64, dv=128), 3), (dict(d=192, dv=64), 3),
    (dict(d=256, dv=128), 3), (dict(d=0, dv=0), 3), (dict(causal=2), 3),
    (dict(Nk=(1 << 30) // 192 + 1), 3), (dict(Nq=(1 << 30) // 192 + 1), 3),
    (dict(o=0), 1), (dict(v=0), 1), (dict(Nk=0), 2),
    (dict(v=Vp + 8), 3),
    (dict(o=Kp + 131072), 4),          # inside K only because K rows are 192 wide
    (dict(lse=Op + 131068), 4),        # last dword of O (d_v wide)
    (dict(scale=float("nan")), 5),
    (dict(Nq=0), 0),
])
def test_dv_validation_codes(kw, code):
    assert call_dv(**kw) == code


def test_dv_extents_use_each_buffer_width():
    # just past K's 192-wide extent and O's 128-wide one: no alias; the
    # call then fails only at the device check (or launches nothing: Nq=0)
    assert call_dv(o=Kp + 196608, Nq=0) == 0
    assert call_dv(lse=Op + 131072, Nq=0) == 0
    import torch
    if torch.cuda.is_available():
        return
    assert call_dv(o=Kp + 196608) == 6
    assert call_dv(lse=Op + 131072) == 6
    for d in (64, 128, 256):
        assert call_dv(d=d, dv=d) == 6
    assert call(d=192) == 3   # fa_fwd has d_v = d: (192, 192) has no kernel


# fa_fwd_splitkv: the key-split plan (host arithmetic) and the workspace rules
def plan(B, H, Nq, Nk, dv=128, n=0):
    return fa.splitkv_workspace_bytes(B, H, Nq, Nk, dv, n)


@pytest.mark.parametrize("B,H,Nq,Nk,n", [
    (1, 8, 4096, 8192, 0), (2, 16, 8192, 8192, 0), (1, 16, 128, 65536, 0), (1, 1, 1, 1, 0), (1, 1, 5, 100, 0),
    (1, 2, 300, 1000, 3), (1, 1, 10, 100, 1000), (1, 1, 10, 256, 5), (3, 5, 77, 8191, 7), (1, 1, 1, 1 << 23, 1024),
])
def test_split_plan_covers_the_keys(B, H, Nq, Nk, n):
    nbytes, used = plan(B, H, Nq, Nk, 128, n)
    assert used >= 1
    if n:
        assert used <= n
    # equal ranges of a multiple of 64 keys, the last one non-empty
    keys = -(-Nk // used)
    keys = -(-keys // 64) * 64
    assert (used - 1) * keys < Nk <= used * keys
    assert nbytes == (used * B * H * Nq * (4 * 128 + 4) if used > 1 else 0)


def test_split_plan_auto_choices():
    assert plan(1, 8, 4096, 8192)[1] == 2       # 256 q-tiles -> two ranges of 4096 keys
    assert plan(2, 16, 8192, 8192) == (0, 1)    # 2048 q-tiles: no split
    assert plan(1, 16, 128, 65536)[1] == 32     # 16 q-tiles -> 32 ranges of 2048 keys
    assert plan(1, 16, 128, 2048)[1] == 4       # ranges kept >= 512 keys
    assert plan(1, 1, 1, 1000)[1] == 1
    assert plan(1, 1, 1, 1000, n=2)[1] == 2     # an explicit request is honoured
    for bad in [dict(B=-1), dict(Nk=0), dict(n=-1), dict(n=1025), dict(dv=0), dict(dv=512), dict(Nq=(1 << 23) + 1)]:
        a = {**dict(B=1, H=1, Nq=10, Nk=100, dv=128, n=0), **bad}
        with pytest.raises(fa.FaError):
            plan(a["B"], a["H"], a["Nq"], a["Nk"], a["dv"], a["n"])


WSp = 0x80000000


def call_split(ws=WSp, ws_bytes=1 << 30, n=2, **kw):
    a = {**GOOD, "dv": GOOD["d"], "causal": 0, **kw}
    return fa.fa_fwd_splitkv_raw(kw.get("q", Qp), kw.get("k", Kp), kw.get("v", Vp), kw.get("o", Op),
                                 kw.get("lse", Lp), a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["dv"], a["scale"],
                                 a["causal"], None, 0, 0, 0, n, ws, ws_bytes, 0)


def test_split_workspace_rules():
    need, used = plan(1, 2, 256, 256, 128, 2)
    assert used == 2 and need == 2 * 2 * 256 * 516
    assert call_split(ws=0) == 8                    # NULL with two ranges
    assert call_split(ws_bytes=need - 1) == 8       # too small
    assert call_split(ws=WSp + 8) == 8              # misaligned
    assert call_split(ws=Op + 64) == 4              # overlaps O
    assert call_split(ws=Kp - 16) == 4              # overlaps K
    assert call_split(n=1025) == 3 and call_split(n=-1) == 3
    # B*H*Nq at 2^33 rows: the merge grid at d_v = 256 would pass 2^31 blocks
    assert call_split(B=1 << 12, H=1 << 11, Nq=1 << 10, Nk=1 << 12, d=256, dv=256, n=2, ws_bytes=1 << 62) == 3
    assert call_split(Nq=0) == 0                    # empty problem: no-op
    import torch
    if torch.cuda.is_available():
        return
    assert call_split(ws_bytes=need) == 6           # valid: reaches the device check
    assert call_split(ws=0, ws_bytes=0, n=1) == 6   # one range needs no workspace
    assert call_split(ws=0, ws_bytes=0, n=0) == 6   # auto plan of a 256-key problem: one range


def test_split_noalloc_rules():
    """The no-allocation split checks its plan against the scratch array
    before any HIP call; other arguments follow fa_fwd_splitkv's rules."""
    cap = fa.splitkv_noalloc_max_bytes()
    assert cap == 48 << 20

    def call_na(**kw):
        a = {**GOOD, "dv": GOOD["d"], "causal": 0, "n": 2, **kw}
        return fa.fa_fwd_splitkv_noalloc_raw(kw.get("q", Qp), kw.get("k", Kp), kw.get("v", Vp), kw.get("o", Op),
                                             kw.get("lse", Lp), a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["dv"],
                                             a["scale"], a["causal"], None, 0, 0, 0, a["n"], 0)

    # 16 heads x 8192 queries x 2 ranges x 516 bytes = 135 MB > 48 MiB
    need, used = plan(1, 16, 8192, 8192, 128, 2)
    assert used == 2 and need > cap
    assert call_na(H=16, Nq=8192, Nk=8192) == 9
    assert call_na(o=Qp) == 4 and call_na(q=0) == 1 and call_na(n=1025) == 3
    assert call_na(scale=float("nan")) == 5 and call_na(Nq=0) == 0
    import torch
    if torch.cuda.is_available():
        return
    assert call_na() == 6                            # fits: reaches the device check
    assert call_na(n=1) == 6


# MXFP8 entry: fake buffers
Q8p, QSp, K8p, KSp, VTp, VSp = 0xD0000000, 0xD8000000, 0xE0000000, 0xE8000000, 0xF0000000, 0xF8000000
GOOD_MX = dict(q8=Q8p, qs=QSp, k8=K8p, ks=KSp, vt=VTp, vs=VSp, o=Op, lse=Lp,
               B=1, H=2, Nq=256, Nk=200, d=128, ldv=256, scale=0.088, causal=0)


def call_mx(**kw):
    a = {**GOOD_MX, **kw}
    return fa.load_library().fa_fwd_mxfp8(a["q8"], a["qs"], a["k8"], a["ks"], a["vt"], a["vs"], a["o"], a["lse"],
                                          a["B"], a["H"], a["Nq"], a["Nk"], a["d"], a["ldv"],
                                          ctypes.c_float(a["scale"]), a["causal"], None)


@pytest.mark.parametrize("kw,code", [
    (dict(q8=0), 1), (dict(vs=0), 1), (dict(lse=0), 1),
    (dict(Nk=0), 2), (dict(B=-1), 2),
    (dict(d=64), 3), (dict(ldv=192), 3), (dict(ldv=100), 3), (dict(ldv=(1 << 24) + 64), 3), (dict(causal=3), 3),
    (dict(qs=QSp + 2), 3), (dict(ks=KSp + 4), 3), (dict(vt=VTp + 8), 3),
    (dict(o=Q8p), 4), (dict(lse=VSp), 4),
    (dict(scale=float("inf")), 5),
    (dict(Nq=0), 0),
])
def test_mxfp8_validation_codes(kw, code):
    assert call_mx(**kw) == code


def test_mxfp8_quantize_validation_codes():
    lib = fa.load_library()
    assert lib.fa_mxfp8_quantize_rows(Qp, Q8p, QSp, 1, 2, 256, 64, 256, None) == 3      # d must be 128
    assert lib.fa_mxfp8_quantize_rows(Qp, Q8p, QSp, 1, 2, 256, 128, 100, None) == 2     # ldS < N
    assert lib.fa_mxfp8_quantize_rows(Qp + 2, Q8p, QSp, 1, 2, 256, 128, 256, None) == 3
    assert lib.fa_mxfp8_quantize_rows(Qp, Qp, QSp, 1, 2, 256, 128, 256, None) == 4      # E overlaps X
    assert lib.fa_mxfp8_quantize_rows(Qp, Q8p, QSp, 1, 2, 0, 128, 0, None) == 0         # empty
    assert lib.fa_mxfp8_quantize_vt(Vp, VTp, VSp, 1, 2, 200, 128, 224, None) == 3       # ldv not a multiple of 64
    assert lib.fa_mxfp8_quantize_vt(Vp, VTp, VSp, 1, 2, 300, 128, 256, None) == 3       # ldv < Nk
    assert lib.fa_mxfp8_quantize_vt(Vp, Vp, VSp, 1, 2, 200, 128, 256, None) == 4


def test_bwd_head_size_256_reaches_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch on fake pointers")
    assert call_bwd(d=256) == 6
    assert call_bwd_dv(hd=256, hdv=256) == 6


def test_bwd_head_size_256_with_a_bias_reaches_the_device_check():
    import torch
    if torch.cuda.is_available():
        pytest.skip("would launch on fake pointers")
    assert call_bwd_bias(d=256) == 6
    assert fa.fa_bwd_dv_raw(Qp, Kp, Vp, Op2, dOp, Lp, dQp, dKp, dVp, Dp, 1, 2, 256, 256, 256, 256, 0.0625, 0,
                            BIASp, 0, 0, 256, 0) == 6
