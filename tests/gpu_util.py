"""Helpers shared by the GPU parity tests: moving stored workload arrays to the
device and measuring errors against the fp64 oracle."""
import numpy as np
import torch

import workloads as G

# tolerances: max |gpu - oracle| / max |oracle| per output tensor
TOL = {G.F32: 1e-4, G.BF16: 2e-2}
# lse is compared as an absolute difference (natural-log units)
LSE_TOL = {G.F32: 1e-4, G.BF16: 2e-2}


def to_dev(a, dtype):
    """numpy storage (fp32 array or bf16 bit patterns) -> CUDA tensor."""
    if dtype == G.BF16:
        t = torch.from_numpy(np.ascontiguousarray(a).view(np.int16)).view(torch.bfloat16)
    else:
        t = torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32))
    return t.cuda()


def to_host64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


def rel_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    assert got.shape == ref.shape, (got.shape, ref.shape)
    assert np.all(np.isfinite(got)), "non-finite GPU output"
    scale = np.max(np.abs(ref))
    if scale == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref)) / scale)


def lse_err(got, ref):
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    both_inf = np.isneginf(got) & np.isneginf(ref)
    assert np.all(np.isneginf(got) == np.isneginf(ref)), "empty-row lse mismatch"
    with np.errstate(invalid="ignore"):
        d = np.abs(np.where(both_inf, 0.0, got - ref))
    return float(np.max(d)) if d.size else 0.0


def dtype_torch(dtype):
    return torch.bfloat16 if dtype == G.BF16 else torch.float32


def elem_rel_err(got, ref, floor=1e-3):
    """Largest elementwise relative error with a floor: max |g - r| / max(|r|,
    floor * max|r|) (reported next to the infinity-norm figure; elementwise
    relative error alone is ill-posed where the reference is near zero)."""
    got, ref = np.asarray(got, np.float64), np.asarray(ref, np.float64)
    scale = np.max(np.abs(ref))
    if scale == 0:
        return float(np.max(np.abs(got)))
    return float(np.max(np.abs(got - ref) / np.maximum(np.abs(ref), floor * scale)))
