"""GPU parity of the decode step (dilated cache + raw ring) and its
consistency with prefill."""
import math

import numpy as np
import pytest
import torch

import dilated_sparse_attention_amd as rat
from dilated_sparse_attention_amd import inputs
from oracle import oracle
from tests.oracle_pins import decode_caches_from_prefill
from tests.parity import announce, assert_parity, guarded_empty, requires_gpu, to_f64

pytestmark = [pytest.mark.gpu, requires_gpu]


def _decode_inputs(B, H, d, nd_cap, w_cap, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    mk = lambda *s: torch.randn(s, generator=g).to(dtype)  # noqa: E731
    return mk(B, H, d), mk(B, H, nd_cap, d), mk(B, H, nd_cap, d), mk(B, H, max(w_cap, 1), d), \
        mk(B, H, max(w_cap, 1), d)


CASES = [
    # (B, T, H, d, D, W, dtype)
    (2, 1, 2, 128, [64, 1], [64, 0], torch.bfloat16),          # first token
    (3, 50, 2, 128, [64, 16], [64, 8], torch.bfloat16),        # T < W, D > T
    (4, 4097, 3, 128, [64, 16, 1], [64, 0, 32], torch.bfloat16),
    (8, 32768, 2, 64, [64, 16], [64, 64], torch.bfloat16),
    (1, 100000, 2, 128, [1, 3], [0, 100], torch.bfloat16),     # few pairs, long cache: split keys
    (2, 300, 2, 64, [4, 300], [10, 0], torch.float32),
    (1, 20000, 1, 128, [1], [7], torch.float32),               # split keys, fp32
]


def run_case(B, T, H, d, D, W, dtype, seed=0):
    nd_cap = max((T + Dh - 1) // Dh for Dh in D) + 2
    w_cap = max(min(Wh, T) for Wh in W) + 1
    q, kd, vd, kw, vw = _decode_inputs(B, H, d, nd_cap, w_cap, dtype, seed)
    dev = [t.cuda() for t in (q, kd, vd, kw, vw)]
    out, check = guarded_empty(q.shape, dtype)
    announce("decode", (B, T, H, d), "D", D, "W", W, dtype)
    rat.dilated_attn_decode(*dev, T=T, D=D, W=W, out=out)
    torch.cuda.synchronize()
    check()
    want = oracle.attn_decode(q, kd, vd, kw, vw, T, D, W, 1 / math.sqrt(d))
    assert_parity(out, want, dtype, "decode out")


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}D{c[4]}W{c[5]}{str(c[6])[6:]}")
def test_decode_parity(case):
    run_case(*case)


def test_decode_ring_order_and_unused_slots():
    """Ring slot order is immaterial; entries past the valid counts are
    never read (NaN there must not leak)."""
    B, T, H, d = 4, 5000, 2, 128
    D, W = [64, 16], [64, 10]
    q, kd, vd, kw, vw = (t.cuda() for t in _decode_inputs(B, H, d, 400, 70, torch.bfloat16, 4))
    announce("decode ring order")
    base = rat.dilated_attn_decode(q, kd, vd, kw, vw, T, D, W)
    perm = torch.randperm(64)
    kw2, vw2 = kw.clone(), vw.clone()
    kw2[:, 0, :64] = kw[:, 0, perm]
    vw2[:, 0, :64] = vw[:, 0, perm]
    for h in range(H):
        nd = (T + D[h] - 1) // D[h]
        kd[:, h, nd:] = float("nan")
        vd[:, h, nd:] = float("nan")
        kw2[:, h, min(W[h], T):] = float("nan")
        vw2[:, h, min(W[h], T):] = float("nan")
    got = rat.dilated_attn_decode(q, kd, vd, kw2, vw2, T, D, W)
    torch.cuda.synchronize()
    assert torch.isfinite(got.float()).all()
    assert (got.float() - base.float()).abs().max().item() <= 2e-2


def test_decode_matches_prefill_last_row():
    """Decode at context T equals the GPU prefill's row T-1 when the caches
    hold the GPU scan's states (dilated) and the raw tokens (ring)."""
    B, T, H, d = 2, 1500, 3, 128
    D, W = [16, 64, 1], [32, 64, 0]
    x = inputs.make_random_prefill(B, T, H, d, torch.bfloat16, 21)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    announce("decode vs prefill")
    ks, vs = rat.scan_prefill(k, v, g)
    pre = rat.dilated_attn_prefill(q, ks, vs, k, v, D=D, W=W)
    rng = np.random.default_rng(0)
    nd_cap = max((T + Dh - 1) // Dh for Dh in D)
    w_cap = max(min(Wh, T) for Wh in W)
    kd, vd, kw, vw = decode_caches_from_prefill(to_f64(ks), to_f64(vs), to_f64(k), to_f64(v), T, D, W,
                                                nd_cap, w_cap, rng)
    cast = lambda a: torch.from_numpy(a).to(torch.bfloat16).cuda().contiguous()  # noqa: E731 (exact)
    out = rat.dilated_attn_decode(q[:, T - 1].contiguous(), cast(kd), cast(vd), cast(kw), cast(vw), T, D, W)
    torch.cuda.synchronize()
    np.testing.assert_allclose(to_f64(out), to_f64(pre[:, T - 1]), rtol=0, atol=2e-2)
    want = oracle.attn_decode(x["q"][:, T - 1], kd, vd, kw, vw, T, D, W, 1 / math.sqrt(d))
    assert_parity(out, want, torch.bfloat16, "decode vs oracle")


@pytest.mark.slow
@pytest.mark.parametrize("w", inputs.DECODE_WORKLOADS, ids=lambda w: w.name)
def test_decode_full_size(w):
    """The full decode workloads in the benchmark's launch configuration,
    every output element against the oracle."""
    x = inputs.make_decode(w, seed=0)
    dev = {n: t.cuda() for n, t in x.items()}
    announce("decode full size", w.name)
    out = rat.dilated_attn_decode(dev["q"], dev["kd"], dev["vd"], dev["kw"], dev["vw"], w.T, list(w.D), list(w.W))
    torch.cuda.synchronize()
    want = oracle.attn_decode(x["q"], x["kd"], x["vd"], x["kw"], x["vw"], w.T, w.D, w.W, w.scale)
    assert_parity(out, want, w.dtype, w.name)
