"""GPU parity of rat_layer_prefill: the recurrence and the attention in one
call, with the states written once into the per-residue history that a
decode loop reads (kc, vc), the raw ring of the last W tokens (kw, vw) and
the fp32 states at T-1.  Every output is checked against the oracle: the
layer output against its fp64 recurrence and attention, the history rows
against its states (rows the call must not write keep a sentinel), the ring
against the raw inputs exactly, and a decode loop continued from the caches
against the oracle's prefill rows at the later positions."""
import math

import numpy as np
import pytest
import torch

import dilated_sparse_attention_amd as rat
from dilated_sparse_attention_amd import inputs
from oracle import oracle
from tests.parity import FP32_ATOL, FP32_RTOL, announce, assert_parity, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]

SENTINEL = 7.0  # exactly representable in bf16 and fp32, far from any state

CASES = [
    # (B, T, H, d, D per head, W per head, L (None: T), mode, dtype)
    (1, 300, 3, 128, [1, 4, 16], [0, 8, 0], None, rat.RESTART, torch.bfloat16),     # full recurrence
    (2, 257, 2, 64, [16, 7], [16, 5], 64, rat.RESTART, torch.bfloat16),               # RESTART, two heads per row
    (1, 700, 2, 128, [64, 20], [128, 33], 64, rat.SLIDING, torch.bfloat16),           # the L = 64 sliding kernel
    (1, 200, 2, 64, [3, 5], [0, 4], 50, rat.SLIDING, torch.bfloat16),                 # general sliding window
    (1, 2048, 4, 128, [1, 1, 64, 64], [0, 0, 256, 256], None, rat.RESTART, torch.bfloat16),  # head-wise hybrid
    (1, 40, 2, 128, [64, 100], [0, 3], None, rat.RESTART, torch.bfloat16),            # D > T
    (2, 1, 2, 128, [1, 16], [4, 0], None, rat.RESTART, torch.bfloat16),               # one token
    (1, 256, 2, 64, [4, 4], [0, 0], None, rat.RESTART, torch.float32),                # the tiny fp32 shape
    (1, 200, 3, 128, [1, 5, 64], [0, 7, 100], 33, rat.SLIDING, torch.float32),
]


def _hist_rows(T, Dh, n_cap):
    p = np.arange(T)
    return (p % Dh) * (n_cap // Dh) + p // Dh


def _ring_positions(T, Wh, w_cap):
    """Position held by each ring slot after a T-token prefill (-1: none)."""
    pos = np.full(w_cap, -1)
    for s in range(min(Wh, w_cap)):
        p = (T - 1) - ((T - 1 - s) % Wh)
        pos[s] = p if p >= 0 else -1
    return pos


def run_case(B, T, H, d, D, W, L, mode, dtype, seed=0):
    Lr = T if L is None else L
    x = inputs.make_random_prefill(B, T, H, d, dtype, seed=seed, gate_mean=1.5)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    n_cap = rat.history_rows(T, D) + 2 * max(D)  # room the call must leave alone
    any_w = any(w > 0 for w in W)
    w_cap = max(W) + 3 if any_w else 0
    kc = torch.full((B, H, n_cap, d), SENTINEL, dtype=dtype, device="cuda")
    vc = torch.full_like(kc, SENTINEL)
    kw = torch.full((B, H, w_cap, d), SENTINEL, dtype=dtype, device="cuda") if any_w else None
    vw = torch.full_like(kw, SENTINEL) if any_w else None
    sliding = mode == rat.SLIDING and Lr < T
    announce("layer prefill", (B, T, H, d), "D", D, "W", W, "L", L, "mode", mode, dtype)
    out, kc, vc, kw, vw, st = rat.layer_prefill(q, k, v, g, D, W, L=Lr, mode=mode, n_cap=n_cap, w_cap=w_cap,
                                                 final_state=not sliding, kc=kc, vc=vc, kw=kw, vw=vw)
    torch.cuda.synchronize()
    ks, vs = oracle.scan(x["k"], x["v"], x["gate"], Lr, mode)
    want = oracle.attn_prefill(x["q"], ks, vs, x["k"] if any_w else None, x["v"] if any_w else None, D, W,
                               1 / math.sqrt(d))
    assert_parity(out, want, dtype, "layer output")
    kc_h, vc_h = kc.cpu(), vc.cpu()
    for h, Dh in enumerate(D):
        rows = _hist_rows(T, Dh, n_cap)
        assert_parity(kc_h[:, h, rows], ks[:, :, h], dtype, f"k history head {h}")
        assert_parity(vc_h[:, h, rows], vs[:, :, h], dtype, f"v history head {h}")
        rest = np.setdiff1d(np.arange(n_cap), rows)
        assert (kc_h[:, h, rest] == SENTINEL).all() and (vc_h[:, h, rest] == SENTINEL).all(), f"head {h}"
    if any_w:
        kw_h, vw_h = kw.cpu(), vw.cpu()
        for h, Wh in enumerate(W):
            pos = _ring_positions(T, Wh, w_cap) if Wh > 0 else np.full(w_cap, -1)
            for s, p in enumerate(pos):
                if p >= 0:
                    assert torch.equal(kw_h[:, h, s], x["k"][:, p, h]), (h, s)
                    assert torch.equal(vw_h[:, h, s], x["v"][:, p, h]), (h, s)
                else:
                    assert (kw_h[:, h, s] == SENTINEL).all() and (vw_h[:, h, s] == SENTINEL).all(), (h, s)
    if not sliding:
        ref = np.stack([ks[:, T - 1], vs[:, T - 1]], axis=2)  # [B,H,2,d]
        got = st.cpu().double().numpy()
        err = np.abs(got - ref)
        assert (err <= FP32_RTOL * np.abs(ref) + FP32_ATOL).all(), f"final state: max err {err.max():.3g}"


@pytest.mark.parametrize("case", CASES,
                         ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}D{c[4]}W{c[5]}L{c[6]}m{c[7]}{str(c[8])[6:]}")
def test_layer_prefill_parity(case):
    run_case(*case)


def test_layer_prefill_matches_two_calls():
    """The one-call layer equals scan_prefill then dilated_attn_prefill
    bit for bit (same kernels' arithmetic, states read from another layout)."""
    B, T, H, d = 2, 1000, 4, 128
    D, W = [16, 16, 1, 64], [0, 64, 0, 128]
    x = inputs.make_random_prefill(B, T, H, d, torch.bfloat16, seed=4, gate_mean=2.0)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    announce("layer prefill vs two calls")
    out1 = rat.layer_prefill(q, k, v, g, D, W)[0]
    ks, vs = rat.scan_prefill(k, v, g)
    out2 = rat.dilated_attn_prefill(q, ks, vs, k, v, D=D, W=W)
    torch.cuda.synchronize()
    assert torch.equal(out1, out2)


@pytest.mark.parametrize("L", [None, 16])
def test_prefill_then_decode_loop(L):
    """A decode loop continued from the caches rat_layer_prefill emitted:
    every step's output is the oracle's prefill output at that position."""
    B, T0, steps, H, d = 2, 300, 20, 3, 128
    D, W = [1, 16, 64], [0, 8, 64]
    Tt = T0 + steps
    Lr = Tt if L is None else L
    x = inputs.make_random_prefill(B, Tt, H, d, torch.bfloat16, seed=8, gate_mean=1.5)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    n_cap = rat.history_rows(Tt, D)
    announce("prefill then decode", "L", L)
    pre = [t[:, :T0].contiguous() for t in (q, k, v, g)]
    _, kc, vc, kw, vw, state = rat.layer_prefill(*pre, D, W, L=min(Lr, T0), n_cap=n_cap)
    wk, wv = oracle.scan(x["k"], x["v"], x["gate"], Lr, 0)
    rows = np.array([(b, t, h) for t in range(T0, Tt) for b in range(B) for h in range(H)], np.int32)
    want = oracle.attn_prefill_rows(x["q"], wk, wv, x["k"], x["v"], rows, D, W, 1 / math.sqrt(d))
    want = want.reshape(steps, B, H, d)
    got = []
    for T in range(T0 + 1, Tt + 1):
        t = T - 1
        out = rat.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                              g[:, t].contiguous(), state, kc, vc, kw, vw, T, D, W, L=Lr)
        got.append(out.clone())
    torch.cuda.synchronize()
    assert_parity(torch.stack(got), want, torch.bfloat16, "decode after layer prefill")


@pytest.mark.slow
@pytest.mark.parametrize("w", [inputs.PREFILL_1P5B, inputs.PREFILL_LONG, inputs.PREFILL_7P6B_HYBRID],
                         ids=lambda w: w.name)
def test_layer_prefill_full_size_sampled(w):
    """The full prefill workloads through the one-call layer (every
    recurrence mode of the workload): sampled output rows against the
    oracle's fp64 recurrence and attention, sampled history rows against
    its states."""
    x = inputs.make_prefill(w, seed=0)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    any_w = any(wh > 0 for wh in w.W)
    rng = np.random.default_rng(2)
    n = 1200
    rows = np.stack([rng.integers(0, w.B, n), rng.integers(0, w.T, n), rng.integers(0, w.H, n)], 1)
    edge = [(b, t, h) for b in (0, w.B - 1) for t in (0, 1, w.T - 1) for h in (0, w.H - 1)]
    rows = np.concatenate([rows, np.array(edge)], 0)
    for mode in w.modes:
        announce("layer prefill full size", w.name, "mode", mode)
        out, kc, vc, _, _, _ = rat.layer_prefill(q, k, v, g, list(w.D), list(w.W), L=w.L, mode=mode,
                                                 final_state=False)
        torch.cuda.synchronize()
        ks, vs = oracle.scan(x["k"], x["v"], x["gate"], w.L, mode)
        want = oracle.attn_prefill_rows(x["q"], ks, vs, x["k"] if any_w else None, x["v"] if any_w else None,
                                        rows, w.D, w.W, w.scale)
        assert_parity(out[rows[:, 0], rows[:, 1], rows[:, 2]], want, w.dtype, f"{w.name} mode {mode}")
        n_cap = kc.shape[2]
        Dr = np.array(w.D)[rows[:, 2]]
        hrow = (rows[:, 1] % Dr) * (n_cap // Dr) + rows[:, 1] // Dr
        b_, t_, h_ = (torch.from_numpy(rows[:, i]) for i in range(3))
        hr = torch.from_numpy(hrow)
        assert_parity(kc.cpu()[b_, h_, hr], ks[rows[:, 0], rows[:, 1], rows[:, 2]], w.dtype, "k history rows")
        assert_parity(vc.cpu()[b_, h_, hr], vs[rows[:, 0], rows[:, 1], rows[:, 2]], w.dtype, "v history rows")
        del out, kc, vc
