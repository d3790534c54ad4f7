"""Helpers shared by the GPU parity tests (no arithmetic of the layer lives here)."""

import os
import sys

import numpy as np
import pytest

TOL_F32 = 1e-4      # max-abs error vs the fp64 oracle, fp32 tensors
TOL_BF16 = 2e-2     # max-abs error vs the fp64 oracle, bf16 outputs with fp32 accumulation


def need_gpu():
    import torch
    if not torch.cuda.is_available():
        pytest.skip("no GPU")


def say(*a):
    print("[case]", *a, flush=True)
    sys.stdout.flush()


def host64(t):
    """torch tensor (any float dtype, any device) -> float64 numpy, exactly."""
    return t.detach().float().cpu().numpy().astype(np.float64)


def maxabs(a, b):
    a = np.asarray(a, dtype=np.float64)
    b = np.asarray(b, dtype=np.float64)
    assert a.shape == b.shape, (a.shape, b.shape)
    assert np.all(np.isfinite(a)), "non-finite values in the GPU result"
    return float(np.max(np.abs(a - b))) if a.size else 0.0


def threads():
    return max(1, min(16, len(os.sched_getaffinity(0))))
