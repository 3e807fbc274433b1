"""Shared helpers of the GPU parity tests: tolerances and case reporting.

Tolerances (elementwise, against the fp64 oracle on the same inputs):
  fp32: |y - r| <= 1e-4 * |r| + 1e-6
  bf16: |y - r| <= 2e-2
The 1e-6 floor covers exact zeros; bf16 outputs are compared per stage
(scan alone; attention fed with the GPU's own bf16 states) and end to end.
"""
from __future__ import annotations

import sys

import numpy as np
import pytest
import torch

FP32_RTOL = 1e-4
FP32_ATOL = 1e-6
BF16_ATOL = 2e-2


def gpu_available():
    return torch.cuda.is_available()


requires_gpu = pytest.mark.skipif(not gpu_available(), reason="needs an MI355X GPU")


def announce(*parts):
    """Name the case before a GPU step (flushed, so a fault still shows it)."""
    print("[case]", *parts, file=sys.stderr, flush=True)


def to_f64(t):
    return t.detach().to("cpu").double().numpy()


def assert_parity(got, want, dtype, what=""):
    """got: torch tensor (any device) or ndarray; want: fp64 ndarray."""
    g = to_f64(got) if hasattr(got, "detach") else np.asarray(got, np.float64)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite output"
    err = np.abs(g - w)
    if dtype == torch.float32:
        bound = FP32_RTOL * np.abs(w) + FP32_ATOL
    else:
        bound = np.full_like(w, BF16_ATOL)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(
            f"{what}: {int(bad.sum())} of {bad.size} elements out of tolerance "
            f"(max err {err.max():.3g}, max |ref| {np.abs(w).max():.3g}); first at {idx.tolist()}")
    return float(err.max()), float(np.abs(w).max())


def guarded_empty(shape, dtype, device="cuda", guard=4096, fill=0x5A):
    """An output tensor sitting between two guard regions of known bytes;
    returns (tensor, check) where check() asserts the guards are intact."""
    n = int(np.prod(shape))
    esz = torch.tensor([], dtype=dtype).element_size()
    gel = guard // esz
    flat = torch.empty(n + 2 * gel, dtype=dtype, device=device)
    flat.view(torch.uint8).fill_(fill)
    out = flat[gel:gel + n].view(shape)

    def check():
        raw = flat.view(torch.uint8).cpu()
        gb = gel * esz
        head, tail = raw[:gb], raw[gb + n * esz:]
        assert bool((head == fill).all()) and bool((tail == fill).all()), "write outside the output tensor"

    return out, check
