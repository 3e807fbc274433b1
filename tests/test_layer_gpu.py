"""End to end: recurrence then attention on the GPU against the oracle's
fp64 states and attention (reduced sizes of every prefill workload)."""
import numpy as np
import pytest
import torch

import dilated_sparse_attention_amd as rat
from dilated_sparse_attention_amd import inputs
from oracle import oracle
from tests.parity import announce, assert_parity, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


# (workload, reduced B, reduced T): the workloads' heads, windows, dtypes
# and distributions at lengths the oracle finishes in seconds
REDUCED = [
    (inputs.TINY_FP32, 1, 256),
    (inputs.PREFILL_1P5B, 1, 1024),
    (inputs.PREFILL_LONG, 1, 1500),
    (inputs.PREFILL_7P6B_HYBRID, 1, 1100),
]


@pytest.mark.parametrize("w,B,T", REDUCED, ids=lambda x: getattr(x, "name", str(x)))
def test_layer_end_to_end(w, B, T):
    x = inputs.make_prefill(w, seed=0, B=B, T=T)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    need_raw = any(wh > 0 for wh in w.W)
    L = min(w.L, T) if w.L < w.T else T
    for mode in w.modes:
        announce("layer", w.name, "B", B, "T", T, "mode", mode)
        out = rat.prefill_two_calls(q, k, v, g, D=list(w.D), W=list(w.W), L=L, mode=mode)
        torch.cuda.synchronize()
        ks, vs = oracle.scan(x["k"], x["v"], x["gate"], L, mode)
        want = oracle.attn_prefill(x["q"], ks, vs, x["k"] if need_raw else None, x["v"] if need_raw else None,
                                   w.D, w.W, w.scale)
        err, ref = assert_parity(out, want, w.dtype, f"{w.name} mode {mode}")
        print(f"{w.name} mode {mode}: max err {err:.3g}, max |ref| {ref:.3g}")
