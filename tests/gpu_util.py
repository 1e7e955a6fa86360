"""Helpers for the GPU tests (no test functions here)."""

import sys

import numpy as np
import torch


def say(*a):
    """Name the case before a GPU step, flushed, so a lost box still shows it."""
    print("[gpu-case]", *a, file=sys.stderr, flush=True)


def bits(t):
    """Raw bit patterns of a device tensor as NumPy (uint32 for fp32, uint16 otherwise)."""
    t = t.detach().contiguous()
    if t.dtype == torch.float32:
        return t.view(torch.int32).cpu().numpy().view(np.uint32)
    return t.view(torch.int16).cpu().numpy().view(np.uint16)


def f64(t):
    return t.detach().float().cpu().numpy().astype(np.float64)


TOL = {"f32": 1e-5, "bf16": 2e-2, "f16": 2e-2}


def max_abs_err(got, ref, rows=None):
    if rows is not None:
        got, ref = got[rows], ref[rows]
    assert np.all(np.isfinite(got)), "non-finite output"
    return float(np.max(np.abs(got - ref))) if got.size else 0.0
