"""MI355X (gfx950) fused attention forward: Python binding of ``libfa06.so``.

``fa_fwd(q, k, v, scale=None) -> (o, lse)`` computes exact, dense
scaled-dot-product attention, ``O = softmax_row(scale * Q K^T + B) V``, plus
the natural-log log-sum-exp of each row ("FlashAttention'ı Anlamak Bölüm 1",
section 0.2, score and output equations), where the optional mask/bias term
B is a causal mask and/or an fp32 additive bias.  Tensors
are BF16 ``[B, H, N, 128]`` on an MI355X; the work runs in the HIP kernel of
``libfa06.so``.  This module only marshals arguments: PyTorch provides device
memory and the current stream.  There is no fallback: if the library is
missing or the device is not gfx950 the call raises.
"""
from __future__ import annotations

import ctypes
import math
import os

_PKG_DIR = os.path.dirname(os.path.abspath(__file__))
LIB_PATH = os.path.join(_PKG_DIR, "libfa06.so")

FA_HEAD_DIM = 128
FA_MAX_SEQ = 1 << 23

STATUS = {
    0: "FA_OK", 1: "FA_ERR_NULL_POINTER", 2: "FA_ERR_INVALID_SHAPE", 3: "FA_ERR_UNSUPPORTED",
    4: "FA_ERR_ALIAS", 5: "FA_ERR_INVALID_SCALE", 6: "FA_ERR_DEVICE", 7: "FA_ERR_LAUNCH",
    8: "FA_ERR_WORKSPACE",
    9: "FA_ERR_SCRATCH",
}


class FaError(RuntimeError):
    """A non-zero status returned by the C ABI."""

    def __init__(self, status: int, message: str):
        super().__init__(f"{message} (status {status})")
        self.status = status


_lib = None


def load_library(path: str | None = None):
    """Load ``libfa06.so`` (built in-tree by ``build.py``); raise if absent.

    torch is imported first so the process has a single HIP runtime: the
    library's dependency on ``libamdhip64.so.7`` then resolves to the copy
    torch already loaded.
    """
    global _lib
    if _lib is not None and path is None:
        return _lib
    import torch  # noqa: F401  (loads the HIP runtime torch uses)

    p = path or LIB_PATH
    if not os.path.exists(p):
        raise ImportError(f"{p} is not built; run `python -m flashattention_forward_06_amd.build` "
                          "or __graft_entry__.build() first")
    lib = ctypes.CDLL(p)
    vp, i64 = ctypes.c_void_p, ctypes.c_int64
    lib.fa_fwd.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float, vp]
    lib.fa_fwd.restype = ctypes.c_int
    lib.fa_fwd_masked.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                  ctypes.c_int, vp, i64, i64, i64, vp]
    lib.fa_fwd_masked.restype = ctypes.c_int
    lib.fa_fwd_dv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                              ctypes.c_int, vp, i64, i64, i64, vp]
    lib.fa_fwd_dv.restype = ctypes.c_int
    lib.fa_fwd_splitkv.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                   ctypes.c_int, vp, i64, i64, i64, i64, vp, i64, vp]
    lib.fa_fwd_splitkv.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc.argtypes = [vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                           ctypes.c_int, vp, i64, i64, i64, i64, vp]
    lib.fa_fwd_splitkv_noalloc.restype = ctypes.c_int
    lib.fa_fwd_splitkv_noalloc_max_bytes.argtypes = []
    lib.fa_fwd_splitkv_noalloc_max_bytes.restype = ctypes.c_int64
    lib.fa_fwd_splitkv_workspace_bytes.argtypes = [i64, i64, i64, i64, i64, i64, ctypes.POINTER(ctypes.c_int64)]
    lib.fa_fwd_splitkv_workspace_bytes.restype = ctypes.c_int64
    lib.fa_status_string.argtypes = [ctypes.c_int]
    lib.fa_status_string.restype = ctypes.c_char_p
    lib.fa_build_info.argtypes = []
    lib.fa_build_info.restype = ctypes.c_char_p
    lib.fa_bwd.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                           ctypes.c_int, vp]
    lib.fa_bwd.restype = ctypes.c_int
    lib.fa_bwd_masked.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, ctypes.c_float,
                                  ctypes.c_int, vp, i64, i64, i64, vp]
    lib.fa_bwd_masked.restype = ctypes.c_int
    lib.fa_bwd_dv.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                              ctypes.c_int, vp, i64, i64, i64, vp]
    lib.fa_bwd_dv.restype = ctypes.c_int
    lib.fa_bwd_build_info.argtypes = []
    lib.fa_bwd_build_info.restype = ctypes.c_char_p
    lib.fa_fwd_mxfp8.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, i64, i64, i64, i64, i64, i64, ctypes.c_float,
                                 ctypes.c_int, vp]
    lib.fa_fwd_mxfp8.restype = ctypes.c_int
    lib.fa_mxfp8_quantize_rows.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp]
    lib.fa_mxfp8_quantize_rows.restype = ctypes.c_int
    lib.fa_mxfp8_quantize_vt.argtypes = [vp, vp, vp, i64, i64, i64, i64, i64, vp]
    lib.fa_mxfp8_quantize_vt.restype = ctypes.c_int
    lib.fa_mxfp8_build_info.argtypes = []
    lib.fa_mxfp8_build_info.restype = ctypes.c_char_p
    if path is None:
        _lib = lib
    return lib


def fa_status_string(status: int) -> str:
    return load_library().fa_status_string(int(status)).decode()


def fa_build_info() -> str:
    return load_library().fa_build_info().decode()


def fa_bwd_build_info() -> str:
    return load_library().fa_bwd_build_info().decode()


def fa_bwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, do_ptr: int, lse_ptr: int,
               dq_ptr: int, dk_ptr: int, dv_ptr: int, delta_ptr: int,
               B: int, H: int, Nq: int, Nk: int, d: int, scale: float, causal: int, stream: int) -> int:
    """Direct call of the C ``fa_bwd`` on raw device pointers; returns the status."""
    return load_library().fa_bwd(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr, delta_ptr,
                                 B, H, Nq, Nk, d, ctypes.c_float(scale), int(causal), stream)


def fa_bwd_masked_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, do_ptr: int, lse_ptr: int,
                      dq_ptr: int, dk_ptr: int, dv_ptr: int, delta_ptr: int,
                      B: int, H: int, Nq: int, Nk: int, d: int, scale: float, causal: int,
                      bias_ptr: int | None, sb: int, sh: int, sq: int, stream: int) -> int:
    """Direct call of the C ``fa_bwd_masked`` on raw device pointers; returns the status."""
    return load_library().fa_bwd_masked(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr,
                                        delta_ptr, B, H, Nq, Nk, d, ctypes.c_float(scale), int(causal), bias_ptr,
                                        sb, sh, sq, stream)


def fa_bwd_dv_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, do_ptr: int, lse_ptr: int,
                  dq_ptr: int, dk_ptr: int, dv_ptr: int, delta_ptr: int,
                  B: int, H: int, Nq: int, Nk: int, d: int, dv: int, scale: float, causal: int,
                  bias_ptr: int | None, sb: int, sh: int, sq: int, stream: int) -> int:
    """Direct call of the C ``fa_bwd_dv`` on raw device pointers; returns the status."""
    return load_library().fa_bwd_dv(q_ptr, k_ptr, v_ptr, o_ptr, do_ptr, lse_ptr, dq_ptr, dk_ptr, dv_ptr,
                                    delta_ptr, B, H, Nq, Nk, d, dv, ctypes.c_float(scale), int(causal), bias_ptr,
                                    sb, sh, sq, stream)


def fa_fwd_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
               B: int, H: int, Nq: int, Nk: int, d: int, scale: float, stream: int) -> int:
    """Direct call of the C ``fa_fwd`` on raw device pointers; returns the status."""
    return load_library().fa_fwd(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, d,
                                 ctypes.c_float(scale), stream)


def fa_fwd_masked_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                      B: int, H: int, Nq: int, Nk: int, d: int, scale: float, causal: int,
                      bias_ptr: int | None, sb: int, sh: int, sq: int, stream: int) -> int:
    """Direct call of the C ``fa_fwd_masked``; returns the status."""
    return load_library().fa_fwd_masked(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, d,
                                        ctypes.c_float(scale), int(causal), bias_ptr, sb, sh, sq, stream)


def fa_fwd_dv_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                  B: int, H: int, Nq: int, Nk: int, d: int, dv: int, scale: float, causal: int,
                  bias_ptr: int | None, sb: int, sh: int, sq: int, stream: int) -> int:
    """Direct call of the C ``fa_fwd_dv``; returns the status."""
    return load_library().fa_fwd_dv(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, d, dv,
                                    ctypes.c_float(scale), int(causal), bias_ptr, sb, sh, sq, stream)


def fa_fwd_splitkv_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                       B: int, H: int, Nq: int, Nk: int, d: int, dv: int, scale: float, causal: int,
                       bias_ptr: int | None, sb: int, sh: int, sq: int, n_splits: int,
                       ws_ptr: int | None, ws_bytes: int, stream: int) -> int:
    """Direct call of the C ``fa_fwd_splitkv``; returns the status."""
    return load_library().fa_fwd_splitkv(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, d, dv,
                                         ctypes.c_float(scale), int(causal), bias_ptr, sb, sh, sq,
                                         int(n_splits), ws_ptr, int(ws_bytes), stream)


def fa_fwd_splitkv_noalloc_raw(q_ptr: int, k_ptr: int, v_ptr: int, o_ptr: int, lse_ptr: int,
                               B: int, H: int, Nq: int, Nk: int, d: int, dv: int, scale: float, causal: int,
                               bias_ptr, sb: int, sh: int, sq: int, n_splits: int, stream: int) -> int:
    """Direct call of the C ``fa_fwd_splitkv_noalloc`` (partials in the
    library's scratch array, no allocation); returns the status."""
    return load_library().fa_fwd_splitkv_noalloc(q_ptr, k_ptr, v_ptr, o_ptr, lse_ptr, B, H, Nq, Nk, d, dv,
                                                 ctypes.c_float(scale), int(causal), bias_ptr, sb, sh, sq,
                                                 int(n_splits), stream)


def splitkv_noalloc_max_bytes() -> int:
    """Size of the scratch array ``fa_fwd_splitkv_noalloc`` uses."""
    return int(load_library().fa_fwd_splitkv_noalloc_max_bytes())


def splitkv_workspace_bytes(B: int, H: int, Nq: int, Nk: int, dv: int, n_splits: int = 0):
    """(bytes, ranges) of the key-split plan ``fa_fwd_splitkv`` uses for these
    sizes; raises FaError on invalid sizes."""
    used = ctypes.c_int64(0)
    n = load_library().fa_fwd_splitkv_workspace_bytes(B, H, Nq, Nk, dv, int(n_splits), ctypes.byref(used))
    if n < 0:
        raise FaError(-n, fa_status_string(-n))
    return int(n), int(used.value)


def _bias_arg(bias, B: int, H: int, Nq: int, Nk: int, device):
    """Bias tensor -> (tensor kept alive, element strides) in the layout the
    library reads: unit key stride and row/head/batch strides that are
    multiples of 4 elements, from a 16-byte aligned base.  Broadcast
    dimensions keep stride 0; anything else is copied once into a padded
    buffer of that layout (argument marshalling, no arithmetic)."""
    import torch

    if not isinstance(bias, torch.Tensor):
        raise TypeError("bias must be a torch.Tensor")
    if bias.dtype != torch.float32:
        raise TypeError(f"bias must be float32, got {bias.dtype}")
    if bias.device != device:
        raise ValueError("bias must be on q's device")
    try:
        full = bias.expand(B, H, Nq, Nk)
    except RuntimeError as e:
        raise ValueError(f"bias of shape {tuple(bias.shape)} does not broadcast to {(B, H, Nq, Nk)}") from e
    st = full.stride()
    ok = (Nk == 1 or st[3] == 1) and all(x >= 0 and x % 4 == 0 for x in st[:3]) and full.data_ptr() % 16 == 0
    if ok:
        return full, st[0], st[1], st[2]
    # copy into [b', h', q', ceil4(Nk)] keeping broadcast dimensions at size 1
    red = [1 if st[i] == 0 else n for i, n in enumerate((B, H, Nq))]
    nk4 = (Nk + 3) // 4 * 4
    buf = torch.zeros(red + [nk4], dtype=torch.float32, device=device)
    buf[..., :Nk].copy_(full[:red[0], :red[1], :red[2]])
    full = buf[..., :Nk].expand(B, H, Nq, Nk)
    st = full.stride()
    return full, st[0], st[1], st[2]


def fa_fwd(q, k, v, scale: float | None = None, out=None, lse=None, causal: bool = False, bias=None,
           n_splits: int | None = None, workspace=None):
    """Fused attention forward on torch tensors.

    q: [B, H, Nq, d] bf16, k: [B, H, Nk, d], v: [B, H, Nk, dv] bf16, all
    contiguous on the same HIP device; (d, dv) is (64, 64), (128, 128),
    (256, 256) or (192, 128).  ``scale`` defaults to 1/sqrt(d).  With
    ``causal``, key j is hidden from query i when j > i + (Nk - Nq).
    ``bias`` (optional) is an fp32 tensor broadcastable to [B, H, Nq, Nk],
    added to the scaled scores.  Rows that see no key (causal with Nq > Nk,
    or a bias of -inf on every key) give O = 0, LSE = -inf.  Returns
    ``(o, lse)``: o [B, H, Nq, dv] bf16 and lse [B, H, Nq] fp32.  Optional
    ``out`` / ``lse`` tensors of those shapes receive the results.  The call is
    enqueued on the current stream of q's device.

    ``n_splits`` (optional) splits every head's keys into ranges computed by
    separate workgroups and merged (``fa_fwd_splitkv``): 0 lets the library
    choose, k >= 1 asks for k ranges.  The fp32 workspace it needs is
    allocated here unless ``workspace`` (a uint8 tensor on q's device of at
    least ``splitkv_workspace_bytes(...)[0]`` bytes) is given.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v)):
        if not isinstance(t, torch.Tensor):
            raise TypeError(f"{name} must be a torch.Tensor")
        if t.dtype != torch.bfloat16:
            raise TypeError(f"{name} must be bfloat16, got {t.dtype}")
        if t.dim() != 4:
            raise ValueError(f"{name} must be 4-D [B, H, N, d], got shape {tuple(t.shape)}")
        if not t.is_cuda:
            raise ValueError(f"{name} must be on a HIP device")
        if not t.is_contiguous():
            raise ValueError(f"{name} must be contiguous")
    if k.device != q.device or v.device != q.device:
        raise ValueError("q, k and v must be on the same device")
    B, H, Nq, d = q.shape
    if k.shape[0] != B or k.shape[1] != H or k.shape[3] != d or tuple(v.shape[:3]) != tuple(k.shape[:3]):
        raise ValueError(f"shape mismatch: q{tuple(q.shape)} k{tuple(k.shape)} v{tuple(v.shape)}")
    Nk = k.shape[2]
    dv = v.shape[3]
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Nq, dv), dtype=torch.bfloat16, device=q.device)
    elif out.dtype != torch.bfloat16 or tuple(out.shape) != (B, H, Nq, dv) or not out.is_contiguous() \
            or out.device != q.device:
        raise ValueError("out must be a contiguous bf16 tensor [B, H, Nq, dv] on q's device")
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=q.device)
    elif lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) or not lse.is_contiguous() \
            or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, Nq] on q's device")
    bias_t, sb, sh, sq = None, 0, 0, 0
    if bias is not None:
        bias_t, sb, sh, sq = _bias_arg(bias, B, H, Nq, Nk, q.device)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    ws_ptr, ws_bytes = None, 0
    if n_splits is not None:
        need, _ = splitkv_workspace_bytes(B, H, Nq, Nk, dv, n_splits)
        if workspace is None and need > 0:
            workspace = torch.empty(need, dtype=torch.uint8, device=q.device)
        if workspace is not None:
            if not isinstance(workspace, torch.Tensor) or workspace.device != q.device or not workspace.is_contiguous():
                raise ValueError("workspace must be a contiguous tensor on q's device")
            ws_ptr, ws_bytes = workspace.data_ptr(), workspace.numel() * workspace.element_size()
    with torch.cuda.device(q.device):
        if n_splits is not None:
            rc = fa_fwd_splitkv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                    B, H, Nq, Nk, d, dv, float(scale), int(bool(causal)),
                                    None if bias_t is None else bias_t.data_ptr(), sb, sh, sq, int(n_splits),
                                    ws_ptr, ws_bytes, stream)
        elif dv != d:
            rc = fa_fwd_dv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                               B, H, Nq, Nk, d, dv, float(scale), int(bool(causal)),
                               None if bias_t is None else bias_t.data_ptr(), sb, sh, sq, stream)
        elif causal or bias_t is not None:
            rc = fa_fwd_masked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                   B, H, Nq, Nk, d, float(scale), int(bool(causal)),
                                   None if bias_t is None else bias_t.data_ptr(), sb, sh, sq, stream)
        else:
            rc = fa_fwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), out.data_ptr(), lse.data_ptr(),
                            B, H, Nq, Nk, d, float(scale), stream)
    if rc != 0:
        raise FaError(rc, fa_status_string(rc))
    return out, lse


def fa_bwd(q, k, v, o, lse, do, scale: float | None = None, causal: bool = False,
           dq=None, dk=None, dv=None, delta=None, bias=None):
    """Attention backward on torch tensors: gradients of a loss through O.

    q, k: bf16 [B, H, N, d], v, o, do: [B, H, N, dv], contiguous on one HIP
    device, (d, dv) one of (64, 64), (128, 128), (256, 256), (192, 128) (o and
    lse are the outputs of ``fa_fwd`` for the same q, k, v, scale, causal
    flag and bias; lse fp32 [B, H, Nq]).  ``bias``: the forward's fp32 bias
    (broadcastable to [B, H, Nq, Nk]); no gradient is formed for it.
    Returns ``(dq, dk, dv)`` in bf16, plus the fp32 ``delta`` workspace
    [B, H, Nq] (D_i = dO_i . O_i) as a fourth value.  Optional output tensors
    of those shapes are written in place.
    """
    import torch

    for name, t in (("q", q), ("k", k), ("v", v), ("o", o), ("do", do)):
        if not isinstance(t, torch.Tensor) or t.dtype != torch.bfloat16 or t.dim() != 4:
            raise TypeError(f"{name} must be a 4-D bfloat16 torch.Tensor")
        if not t.is_cuda or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"{name} must be contiguous on q's HIP device")
    B, H, Nq, d = q.shape
    Nk = k.shape[2]
    dvh = v.shape[3]
    if tuple(k.shape) != (B, H, Nk, d) or tuple(v.shape) != (B, H, Nk, dvh) or tuple(o.shape) != (B, H, Nq, dvh) \
            or tuple(do.shape) != (B, H, Nq, dvh):
        raise ValueError("shape mismatch among q, k, v, o, do")
    if not isinstance(lse, torch.Tensor) or lse.dtype != torch.float32 or tuple(lse.shape) != (B, H, Nq) \
            or not lse.is_contiguous() or lse.device != q.device:
        raise ValueError("lse must be a contiguous fp32 tensor [B, H, Nq] on q's device")
    if scale is None:
        scale = 1.0 / math.sqrt(d)

    def out(t, like, dtype):
        if t is None:
            return torch.empty(like, dtype=dtype, device=q.device)
        if t.dtype != dtype or tuple(t.shape) != tuple(like) or not t.is_contiguous() or t.device != q.device:
            raise ValueError(f"output tensor must be contiguous {dtype} {tuple(like)} on q's device")
        return t

    dq = out(dq, (B, H, Nq, d), torch.bfloat16)
    dk = out(dk, (B, H, Nk, d), torch.bfloat16)
    dv = out(dv, (B, H, Nk, dvh), torch.bfloat16)
    delta = out(delta, (B, H, Nq), torch.float32)
    stream = torch.cuda.current_stream(q.device).cuda_stream
    bias_t, sb, sh, sq = None, 0, 0, 0
    if bias is not None:
        bias_t, sb, sh, sq = _bias_arg(bias, B, H, Nq, Nk, q.device)
    with torch.cuda.device(q.device):
        if dvh != d:
            rc = fa_bwd_dv_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                               lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                               B, H, Nq, Nk, d, dvh, float(scale), int(bool(causal)),
                               None if bias_t is None else bias_t.data_ptr(), sb, sh, sq, stream)
        elif bias_t is not None:
            rc = fa_bwd_masked_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(),
                                   lse.data_ptr(), dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                                   B, H, Nq, Nk, d, float(scale), int(bool(causal)), bias_t.data_ptr(), sb, sh, sq,
                                   stream)
        else:
            rc = fa_bwd_raw(q.data_ptr(), k.data_ptr(), v.data_ptr(), o.data_ptr(), do.data_ptr(), lse.data_ptr(),
                            dq.data_ptr(), dk.data_ptr(), dv.data_ptr(), delta.data_ptr(),
                            B, H, Nq, Nk, d, float(scale), int(bool(causal)), stream)
    if rc != 0:
        raise FaError(rc, fa_status_string(rc))
    return dq, dk, dv, delta


def _attention_function():
    """torch.autograd.Function over fa_fwd / fa_bwd, built on first use (torch
    is imported lazily, as everywhere in this module)."""
    global _AttentionFn
    if _AttentionFn is not None:
        return _AttentionFn
    import torch

    class _Attention(torch.autograd.Function):
        @staticmethod
        def forward(ctx, q, k, v, scale, causal, bias):
            o, lse = fa_fwd(q, k, v, scale=scale, causal=causal, bias=bias)
            ctx.save_for_backward(q, k, v, o, lse)
            ctx.scale, ctx.causal, ctx.bias = scale, causal, bias
            return o

        @staticmethod
        def backward(ctx, do):
            q, k, v, o, lse = ctx.saved_tensors
            dq, dk, dv, _ = fa_bwd(q, k, v, o, lse, do.contiguous(), scale=ctx.scale, causal=ctx.causal,
                                   bias=ctx.bias)
            return dq, dk, dv, None, None, None

    _AttentionFn = _Attention
    return _AttentionFn


_AttentionFn = None


def attention(q, k, v, scale: float | None = None, causal: bool = False, bias=None):
    """Differentiable attention for training: O = softmax(scale Q K^T + bias) V.

    The forward pass is ``fa_fwd`` and the backward pass ``fa_bwd`` (gradients
    by recomputation from the forward's log-sum-exp), both in this library's
    HIP kernels; O and the log-sum-exp are kept for the backward pass.
    q, k: bf16 [B, H, N, d], v: bf16 [B, H, Nk, dv] on one HIP device, (d, dv)
    one of (64, 64), (128, 128), (256, 256), (192, 128).  ``scale``
    defaults to 1/sqrt(d).  No
    gradient flows to ``bias``: pass a bias that does not require one.
    Returns O, bf16 [B, H, Nq, dv].
    """
    import torch

    if bias is not None and isinstance(bias, torch.Tensor) and bias.requires_grad:
        raise NotImplementedError("attention(): no gradient is formed for the bias; pass bias.detach()")
    if scale is None:
        scale = 1.0 / math.sqrt(q.shape[-1])
    return _attention_function().apply(q, k, v, float(scale), bool(causal), bias)


def fa_mxfp8_build_info() -> str:
    return load_library().fa_mxfp8_build_info().decode()


def _check(rc):
    if rc != 0:
        raise FaError(rc, fa_status_string(rc))


def _u8(name, t, shape, device):
    import torch
    if not isinstance(t, torch.Tensor) or t.dtype != torch.uint8 or tuple(t.shape) != tuple(shape) \
            or not t.is_contiguous() or t.device != device:
        raise ValueError(f"{name} must be a contiguous uint8 tensor {tuple(shape)} on {device}")


def mxfp8_quantize_rows(x, ld: int | None = None):
    """bf16 [B, H, N, 128] -> (E4M3 [B, H, N, 128] uint8, E8M0 scales [B, H, ld, 4] uint8)."""
    import torch
    if not isinstance(x, torch.Tensor) or x.dtype != torch.bfloat16 or x.dim() != 4 or not x.is_cuda \
            or not x.is_contiguous():
        raise ValueError("x must be a contiguous 4-D bfloat16 tensor on a HIP device")
    B, H, N, d = x.shape
    ld = N if ld is None else ld
    e = torch.empty((B, H, N, d), dtype=torch.uint8, device=x.device)
    sc = torch.zeros((B, H, ld, d // 32), dtype=torch.uint8, device=x.device)
    with torch.cuda.device(x.device):
        _check(load_library().fa_mxfp8_quantize_rows(x.data_ptr(), e.data_ptr(), sc.data_ptr(), B, H, N, d, ld,
                                                     torch.cuda.current_stream(x.device).cuda_stream))
    return e, sc


def mxfp8_quantize_vt(v, ldv: int | None = None):
    """bf16 V [B, H, Nk, 128] -> (V^T E4M3 [B, H, 128, ldv], E8M0 [B, H, ldv/32, 128]); ldv defaults to
    Nk rounded up to a multiple of 64."""
    import torch
    if not isinstance(v, torch.Tensor) or v.dtype != torch.bfloat16 or v.dim() != 4 or not v.is_cuda \
            or not v.is_contiguous():
        raise ValueError("v must be a contiguous 4-D bfloat16 tensor on a HIP device")
    B, H, Nk, d = v.shape
    ldv = (Nk + 63) // 64 * 64 if ldv is None else ldv
    vt = torch.empty((B, H, d, ldv), dtype=torch.uint8, device=v.device)
    vs = torch.empty((B, H, ldv // 32, d), dtype=torch.uint8, device=v.device)
    with torch.cuda.device(v.device):
        _check(load_library().fa_mxfp8_quantize_vt(v.data_ptr(), vt.data_ptr(), vs.data_ptr(), B, H, Nk, d, ldv,
                                                   torch.cuda.current_stream(v.device).cuda_stream))
    return vt, vs


def mxfp8_inputs(q, k, v):
    """Quantize bf16 q, k, v on the GPU into the arguments of fa_fwd_mxfp8:
    (q8, qs, k8, ks, vt8, vs, Nk)."""
    ldv = (k.shape[2] + 63) // 64 * 64
    q8, qs = mxfp8_quantize_rows(q)
    k8, ks = mxfp8_quantize_rows(k, ld=ldv)
    vt8, vs = mxfp8_quantize_vt(v, ldv=ldv)
    return q8, qs, k8, ks, vt8, vs, k.shape[2]


def fa_fwd_mxfp8(q8, qs, k8, ks, vt8, vs, Nk: int, scale: float | None = None, causal: bool = False,
                 out=None, lse=None):
    """Attention forward on MXFP8 inputs (layouts as returned by mxfp8_inputs).

    Returns ``(o, lse)``: o [B, H, Nq, 128] bf16, lse [B, H, Nq] fp32."""
    import torch
    B, H, Nq, d = q8.shape
    ldv = vt8.shape[3]
    dev = q8.device
    for name, t, shape in (("q8", q8, (B, H, Nq, d)), ("qs", qs, (B, H, Nq, d // 32)),
                           ("k8", k8, (B, H, Nk, d)), ("ks", ks, (B, H, ldv, d // 32)),
                           ("vt8", vt8, (B, H, d, ldv)), ("vs", vs, (B, H, ldv // 32, d))):
        _u8(name, t, shape, dev)
    if scale is None:
        scale = 1.0 / math.sqrt(d)
    if out is None:
        out = torch.empty((B, H, Nq, d), dtype=torch.bfloat16, device=dev)
    if lse is None:
        lse = torch.empty((B, H, Nq), dtype=torch.float32, device=dev)
    with torch.cuda.device(dev):
        _check(load_library().fa_fwd_mxfp8(q8.data_ptr(), qs.data_ptr(), k8.data_ptr(), ks.data_ptr(),
                                           vt8.data_ptr(), vs.data_ptr(), out.data_ptr(), lse.data_ptr(),
                                           B, H, Nq, Nk, d, ldv, float(scale), int(bool(causal)),
                                           torch.cuda.current_stream(dev).cuda_stream))
    return out, lse


__all__ = ["attention", "fa_bwd_dv_raw", "fa_bwd_masked_raw", "fa_fwd_dv_raw", "fa_fwd_mxfp8", "mxfp8_inputs", "mxfp8_quantize_rows", "mxfp8_quantize_vt", "fa_mxfp8_build_info", "fa_bwd", "fa_bwd_raw", "fa_bwd_build_info", "fa_fwd", "fa_fwd_raw", "fa_fwd_masked_raw", "fa_status_string", "fa_build_info", "FaError", "load_library",
           "LIB_PATH", "FA_HEAD_DIM", "FA_MAX_SEQ", "STATUS", "fa_fwd_splitkv_raw", "splitkv_workspace_bytes",
           "fa_fwd_splitkv_noalloc_raw", "splitkv_noalloc_max_bytes"]
