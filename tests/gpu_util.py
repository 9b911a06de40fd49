"""Helpers shared by the GPU parity tests (comparison metrics, device setup)."""
import sys

import numpy as np
import torch

DEV = "cuda:0"

TOL_F32 = 1e-4    # max row-relative error, f32 path
TOL_I8F16 = 3e-3  # max row-relative error, int8-weight / f16-activation path


def row_rel_err(got, ref):
    """max over rows of max_j |got - ref| / max_j |ref| (the row-normwise form of
    max|d|/max|y|)."""
    got = np.asarray(got, np.float64).reshape(ref.shape[0], -1)
    ref = np.asarray(ref, np.float64).reshape(ref.shape[0], -1)
    den = np.abs(ref).max(1)
    den[den == 0] = 1.0
    return float((np.abs(got - ref).max(1) / den).max())


def to_dev(a, dtype=None):
    t = torch.from_numpy(np.ascontiguousarray(a))
    if dtype is not None:
        t = t.to(dtype)
    return t.to(DEV)


def host(t):
    torch.cuda.synchronize()
    return t.float().cpu().numpy().astype(np.float64) if t.dtype == torch.float16 else \
        t.cpu().numpy().astype(np.float64) if t.is_floating_point() else t.cpu().numpy()


def say(*a):
    print(*a, flush=True)
    sys.stdout.flush()
