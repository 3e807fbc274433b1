"""GPU parity of the recurrence (stage 1) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import dilated_sparse_attention_amd as rat
from dilated_sparse_attention_amd import inputs
from oracle import oracle
from tests.parity import announce, assert_parity, guarded_empty, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

CASES = [
    # (B, T, H, d, L, mode, dtype)
    (1, 1, 1, 64, 1, 0, torch.bfloat16),
    (1, 37, 1, 64, 37, 0, torch.bfloat16),        # one partial chunk, half a channel block
    (2, 300, 3, 64, 300, 0, torch.bfloat16),      # ragged chunk, 192 channels
    (1, 1000, 2, 128, 1000, 0, torch.bfloat16),   # 4 chunks, look-back chain
    (3, 2049, 1, 128, 2049, 0, torch.bfloat16),
    (1, 4100, 2, 64, 100, 0, torch.bfloat16),     # RESTART period not aligned to chunks
    (1, 700, 2, 128, 64, 0, torch.bfloat16),      # RESTART at L* = 64
    (1, 700, 2, 128, 7, 0, torch.bfloat16),
    (1, 700, 2, 128, 64, 1, torch.bfloat16),      # SLIDING at L* = 64
    (2, 1000, 3, 64, 64, 1, torch.bfloat16),      # SLIDING L = 64: ragged chunks, 192 channels
    (1, 65, 2, 128, 64, 1, torch.bfloat16),       # one token past the first tile
    (1, 129, 1, 64, 64, 1, torch.bfloat16),       # one token past the first chunk
    (2, 333, 1, 64, 16, 1, torch.bfloat16),
    (1, 200, 1, 64, 1, 1, torch.bfloat16),
    (1, 90, 1, 128, 5, 1, torch.bfloat16),
    (1, 256, 2, 64, 256, 0, torch.float32),       # the tiny fp32 workload's shape
    (2, 513, 2, 64, 513, 0, torch.float32),
    (1, 700, 1, 128, 64, 0, torch.float32),
    (1, 300, 1, 64, 64, 1, torch.float32),
    (1, 129, 3, 64, 10, 1, torch.float32),
]


def run_case(B, T, H, d, L, mode, dtype, seed=0, gate_mean=2.0):
    x = inputs.make_random_prefill(B, T, H, d, dtype, seed, gate_mean=gate_mean)
    k, v, g = (x[n].cuda() for n in ("k", "v", "gate"))
    ks, chk1 = guarded_empty(k.shape, dtype)
    vs, chk2 = guarded_empty(v.shape, dtype)
    announce("scan", (B, T, H, d), "L", L, "mode", mode, dtype, "seed", seed)
    rat.scan_prefill(k, v, g, L=L, mode=mode, k_state=ks, v_state=vs)
    torch.cuda.synchronize()
    chk1()
    chk2()
    wk, wv = oracle.scan(x["k"], x["v"], x["gate"], L, mode)
    assert_parity(ks, wk, dtype, "k_state")
    assert_parity(vs, wv, dtype, "v_state")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}L{c[4]}m{c[5]}{str(c[6])[6:]}")
def test_scan_parity(case):
    run_case(*case)


def test_scan_gate_limits():
    """logit -inf: the state is the input; +inf: the state stays zero."""
    for dtype in (torch.bfloat16, torch.float32):
        B, T, H, d = 1, 600, 2, 64
        x = inputs.make_random_prefill(B, T, H, d, dtype, 3)
        k, v = x["k"].cuda(), x["v"].cuda()
        announce("scan limits", dtype)
        ks, vs = rat.scan_prefill(k, v, torch.full_like(k, -math.inf))
        assert torch.equal(ks, k) and torch.equal(vs, v)
        ks, vs = rat.scan_prefill(k, v, torch.full_like(k, math.inf))
        assert not ks.any() and not vs.any()
        for mode, L in ((0, 64), (1, 64)):
            ks, vs = rat.scan_prefill(k, v, torch.full_like(k, -math.inf), L=L, mode=mode)
            assert torch.equal(ks, k) and torch.equal(vs, v)


def test_scan_repeat_and_workspace_reuse():
    """Calls of different sizes share one workspace (epoch-tagged carries);
    each must match the oracle, a repeated shape included.  Repeats are not
    asserted bit-equal: the decoupled look-back folds a timing-dependent
    number of predecessor aggregates into a chunk's carry, so two runs agree
    only up to fp32 rounding order (and may differ in a bf16 rounding)."""
    shapes = [(1, 3000, 2, 128), (2, 700, 1, 64), (1, 3000, 2, 128), (1, 5000, 4, 64)]
    first = {}
    for i, (B, T, H, d) in enumerate(shapes):
        x = inputs.make_random_prefill(B, T, H, d, torch.bfloat16, 11)
        k, v, g = (x[n].cuda() for n in ("k", "v", "gate"))
        announce("scan reuse", i, (B, T, H, d))
        ks, vs = rat.scan_prefill(k, v, g)
        torch.cuda.synchronize()
        if (B, T, H, d) in first:  # a repeat: within one bf16 rounding of the first run
            diff = (first[(B, T, H, d)].float() - ks.float()).abs()
            assert float(diff.max()) <= 2.0 ** -7 * float(ks.float().abs().max()) + 1e-6
        first[(B, T, H, d)] = ks.clone()
        wk, wv = oracle.scan(x["k"], x["v"], x["gate"], T, 0)
        assert_parity(ks, wk, torch.bfloat16, "k_state")
        assert_parity(vs, wv, torch.bfloat16, "v_state")


@pytest.mark.slow
@pytest.mark.parametrize("w", inputs.PREFILL_WORKLOADS, ids=lambda w: w.name)
def test_scan_full_size(w):
    """Every element of the full-size workloads (each recurrence mode)."""
    x = inputs.make_prefill(w, seed=0)
    k, v, g = (x[n].cuda() for n in ("k", "v", "gate"))
    for mode in w.modes:
        announce("scan full size", w.name, "mode", mode)
        ks, vs = rat.scan_prefill(k, v, g, L=w.L, mode=mode)
        torch.cuda.synchronize()
        wk, wv = oracle.scan(x["k"], x["v"], x["gate"], w.L, mode)
        assert_parity(ks, wk, w.dtype, f"{w.name} k_state")
        assert_parity(vs, wv, w.dtype, f"{w.name} v_state")
        del wk, wv
