"""GPU parity of the layer backward (rat_layer_backward) against the fp64
oracle's backward, which is pinned by central differences of the forward.

The GPU backward takes the forward's saved states as the GPU forward
produced them; the oracle recomputes its own in fp64.  Tolerance, elementwise
per gradient tensor r with got g:
    |g - r| <= rtol * (|r| + rms(r))
  bf16 inputs: rtol = 5e-2.  The saved states are rounded to bf16 (relative
  2^-9); the backward recomputes the softmax from them in fp32 and forms
  <dout, out> from that softmax, so no rounded forward output enters.  The
  gradients are driven by differences of states at nearby positions (a
  query's few keys early in a residue, dp_j - delta): consecutive states
  differ by (1 - g)(x_t - h_{t-1}), so such a difference carries the
  rounding amplified by up to 1/(1 - g), about 8 at the workloads' gate
  mean of 2 (sigmoid(2) = 0.88).  Two such factors give about 3%; 5e-2
  bounds it.  Sums with cancellation make the tensor's RMS the floor.
  fp32 inputs: rtol = 1e-4 (fp32 arithmetic over sums of a few hundred terms).
"""
import math

import numpy as np
import pytest
import torch

import dilated_sparse_attention_amd as rat
from dilated_sparse_attention_amd import inputs
from oracle import oracle
from tests.parity import announce, requires_gpu, to_f64

pytestmark = [pytest.mark.gpu, requires_gpu]

RTOL = {torch.bfloat16: 5e-2, torch.float32: 1e-4}


def assert_grad(got, want, dtype, what):
    g = to_f64(got)
    w = np.asarray(want, np.float64)
    assert g.shape == w.shape, (what, g.shape, w.shape)
    assert np.isfinite(g).all(), f"{what}: non-finite"
    rms = float(np.sqrt(np.mean(w * w))) if w.size else 0.0
    err = np.abs(g - w)
    bound = RTOL[dtype] * (np.abs(w) + rms)
    bad = err > bound
    if bad.any():
        idx = np.argwhere(bad)[:5]
        raise AssertionError(f"{what}: {int(bad.sum())} of {bad.size} out of tolerance (max err {err.max():.3g}, "
                             f"rms {rms:.3g}); first at {idx.tolist()}")
    return float(err.max()), rms


def forward_and_backward(x, D, W, L, mode, dout, dtype):
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    ks, vs = rat.scan_prefill(k, v, g, L=L, mode=mode)
    grads = rat.layer_backward(q, k, v, g, ks, vs, dout.cuda(), D, W, L=L, mode=mode)
    torch.cuda.synchronize()
    return grads


CASES = [
    # (B, T, H, d, D per head, W per head, L (None: T), dtype)
    (1, 200, 3, 128, [1, 4, 16], [0, 8, 0], None, torch.bfloat16),
    (2, 130, 2, 64, [16, 7], [16, 5], 64, torch.bfloat16),       # RESTART every 64, ragged chunks
    (1, 300, 2, 128, [1, 64], [0, 0], 33, torch.bfloat16),        # RESTART cutting inside the 16-token chunks
    (1, 40, 2, 128, [64, 100], [0, 3], None, torch.bfloat16),     # D > T: own state only
    (1, 96, 2, 128, [1, 3], [0, 5], None, torch.float32),
    (2, 77, 2, 64, [5, 1], [2, 0], 20, torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}D{c[4]}W{c[5]}L{c[6]}{str(c[7])[6:]}")
def test_backward_parity(case):
    B, T, H, d, D, W, L, dtype = case
    Lr = T if L is None else L
    x = inputs.make_random_prefill(B, T, H, d, dtype, seed=31, gate_mean=1.5)
    dout = torch.randn((B, T, H, d), generator=torch.Generator().manual_seed(32)).to(dtype)
    announce("backward", case)
    got = forward_and_backward(x, D, W, Lr, rat.RESTART, dout, dtype)
    want = oracle.layer_backward(x["q"], x["k"], x["v"], x["gate"], dout, Lr, 0, D, W, 1 / math.sqrt(d))
    for name, g_, w_ in zip(("dq", "dk", "dv", "dgate"), got, want):
        assert_grad(g_, w_, dtype, name)


def test_backward_deterministic():
    x = inputs.make_random_prefill(1, 300, 2, 128, torch.bfloat16, seed=33)
    dout = torch.randn((1, 300, 2, 128), generator=torch.Generator().manual_seed(34)).to(torch.bfloat16)
    announce("backward determinism")
    a = forward_and_backward(x, [1, 16], [0, 32], 300, rat.RESTART, dout, torch.bfloat16)
    b = forward_and_backward(x, [1, 16], [0, 32], 300, rat.RESTART, dout, torch.bfloat16)
    for ga, gb in zip(a, b):
        assert torch.equal(ga, gb)


@pytest.mark.slow
def test_backward_arl_full_size_sampled():
    """The training workload of Active Recurrence Learning on the 1.5B-scale
    layer (B = 4, T = 4096, H = 16, d = 128, full recurrence): half of the
    batch at D = 1, half at D = 64, one backward call per half.  Sampled
    heads are checked in full against the oracle run on that head alone
    (the attention and the recurrence of a head touch no other head)."""
    w = inputs.PREFILL_1P5B
    x = inputs.make_prefill(w, seed=5)
    dout = (torch.randn((w.B, w.T, w.H, w.d), generator=torch.Generator().manual_seed(6)) * 0.05).to(w.dtype)
    half = w.B // 2
    for (b0, Dv, samples) in [(0, 1, [(1, 3)]), (half, 64, [(0, 0), (1, 15)])]:
        xs = {n: t[b0:b0 + half].contiguous() for n, t in x.items()}
        announce("backward full size", "D", Dv)
        got = forward_and_backward(xs, [Dv] * w.H, [0] * w.H, w.T, rat.RESTART, dout[b0:b0 + half].contiguous(),
                                   w.dtype)
        for (b, h) in samples:
            sl = {n: xs[n][b:b + 1, :, h:h + 1].contiguous() for n in ("q", "k", "v", "gate")}
            want = oracle.layer_backward(sl["q"], sl["k"], sl["v"], sl["gate"],
                                         dout[b0 + b:b0 + b + 1, :, h:h + 1], w.T, 0, [Dv], [0], w.scale)
            for name, g_, w_ in zip(("dq", "dk", "dv", "dgate"), got, want):
                assert_grad(g_[b:b + 1, :, h:h + 1], w_, w.dtype, f"D={Dv} b={b} h={h} {name}")
