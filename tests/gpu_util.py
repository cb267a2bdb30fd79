"""Helpers for the GPU tests: moving bf16 bit arrays to and from the device,
and the parity gates against the fp64 oracle."""
import sys

import numpy as np

# Parity gates against the unrounded fp64 oracle (BF16 output, fp32 LSE).
MAX_ABS_O = 2e-2
MEAN_ABS_O = 2e-3
MAX_ABS_LSE = 1e-3


def say(msg):
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(bits):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).cuda()


def o_to_f64(o):
    import torch
    return o.float().cpu().numpy().astype(np.float64)


def bits_of_tensor(t):
    import torch
    return t.contiguous().view(torch.int16).cpu().numpy().view(np.uint16)


def check_parity(O_gpu, L_gpu, O_ref, L_ref, label=""):
    """Element-wise comparison; returns diagnostics, asserts the gates."""
    dO = np.abs(O_gpu - O_ref)
    dL = np.abs(L_gpu - L_ref)
    diag = dict(max_dO=float(dO.max()) if dO.size else 0.0,
                mean_dO=float(dO.mean()) if dO.size else 0.0,
                max_dLSE=float(dL.max()) if dL.size else 0.0,
                rel_rms=float(np.sqrt((dO ** 2).sum() / max((O_ref ** 2).sum(), 1e-300))) if dO.size else 0.0)
    say(f"  parity {label}: {diag}")
    assert np.all(np.isfinite(O_gpu)) and np.all(np.isfinite(L_gpu)), "non-finite output"
    assert diag["max_dO"] <= MAX_ABS_O, diag
    assert diag["mean_dO"] <= MEAN_ABS_O, diag
    assert diag["max_dLSE"] <= MAX_ABS_LSE, diag
    return diag
