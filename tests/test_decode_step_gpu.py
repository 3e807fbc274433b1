"""GPU parity of the decode loop: prefill hands its fp32 final state to
rat_decode_step, which advances the recurrence one token at a time, appends
to the per-residue state history and the raw ring, and attends.  Every
step's output must equal the oracle's prefill output at that position, and
the running state the oracle's recurrence."""
import math

import numpy as np
import pytest
import torch

import dilated_sparse_attention_amd as rat
from dilated_sparse_attention_amd import inputs
from oracle import oracle
from tests.parity import FP32_ATOL, FP32_RTOL, announce, assert_parity, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _history(ks, vs, T0, D, n_cap):
    """[B,H,n_cap,d] per-residue histories of the first T0 states (row of
    position p: (p mod D[h]) * (n_cap // D[h]) + p // D[h])."""
    B, _, H, d = ks.shape
    kc = torch.zeros((B, H, n_cap, d), dtype=ks.dtype, device=ks.device)
    vc = torch.zeros_like(kc)
    for h, Dh in enumerate(D):
        p = torch.arange(T0, device=ks.device)
        rows = (p % Dh) * (n_cap // Dh) + p // Dh
        kc[:, h, rows] = ks[:, :T0, h]
        vc[:, h, rows] = vs[:, :T0, h]
    return kc, vc


def _ring(k, v, T0, W, w_cap):
    """[B,H,w_cap,d] rings holding raw position p in slot p mod W[h]."""
    B, _, H, d = k.shape
    kw = torch.zeros((B, H, max(w_cap, 1), d), dtype=k.dtype, device=k.device)
    vw = torch.zeros_like(kw)
    for h, Wh in enumerate(W):
        if Wh == 0:
            continue
        p = torch.arange(max(0, T0 - Wh), T0, device=k.device)
        kw[:, h, p % Wh] = k[:, p, h]
        vw[:, h, p % Wh] = v[:, p, h]
    return kw, vw


CASES = [
    # (B, T0, steps, H, d, D, W, L)
    (2, 50, 24, 3, 128, [1, 4, 16], [0, 8, 5], None),          # full recurrence
    (1, 0, 40, 2, 64, [16, 3], [16, 0], None),                 # decoding from the first token
    (2, 60, 30, 2, 128, [64, 5], [64, 7], 16),                  # RESTART every 16 positions
    (1, 1000, 8, 2, 128, [64, 1], [128, 0], None),              # long prefill, split keys on the dense head
]


# every case in bf16; the first and the RESTART one also in fp32 (the step
# kernel's 4-channel vectors and the fp32 decode kernel)
LOOP_CASES = [(c, torch.bfloat16) for c in CASES] + [(CASES[0], torch.float32), (CASES[2], torch.float32)]


@pytest.mark.parametrize("case,dtype", LOOP_CASES,
                         ids=lambda c: f"B{c[0]}T{c[1]}+{c[2]}H{c[3]}d{c[4]}D{c[5]}W{c[6]}L{c[7]}"
                         if isinstance(c, tuple) else str(c)[6:])
def test_decode_loop(case, dtype):
    B, T0, steps, H, d, D, W, L = case
    Tt = T0 + steps
    Lr = Tt if L is None else L
    x = inputs.make_random_prefill(B, Tt, H, d, dtype, seed=3, gate_mean=1.5)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    n_cap = max(Dh * ((Tt + Dh - 1) // Dh) for Dh in D) + 16
    w_cap = max(W) + 3
    state = torch.zeros((B, H, 2, d), dtype=torch.float32, device="cuda")
    if T0 > 0:
        announce("decode loop prefill", case, dtype)
        ks, vs = rat.scan_prefill(k[:, :T0].contiguous(), v[:, :T0].contiguous(), g[:, :T0].contiguous(),
                                  L=min(Lr, T0) if Lr < T0 else T0, final_state=state)
        kc, vc = _history(ks, vs, T0, D, n_cap)
    else:
        kc = torch.zeros((B, H, n_cap, d), dtype=dtype, device="cuda")
        vc = torch.zeros_like(kc)
    kw, vw = _ring(k, v, T0, W, w_cap)

    wk, wv = oracle.scan(x["k"], x["v"], x["gate"], Lr, 0)
    rows = np.array([(b, t, h) for t in range(T0, Tt) for b in range(B) for h in range(H)], np.int32)
    want = oracle.attn_prefill_rows(x["q"], wk, wv, x["k"], x["v"], rows, D, W, 1 / math.sqrt(d))
    want = want.reshape(steps, B, H, d)

    got = []
    for T in range(T0 + 1, Tt + 1):
        announce("decode step", case, "T", T)
        t = T - 1
        out = rat.decode_step(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                              g[:, t].contiguous(), state, kc, vc, kw, vw, T, D, W, L=Lr)
        got.append(out.clone())
    torch.cuda.synchronize()
    assert_parity(torch.stack(got), want, dtype, "decode loop outputs")
    # the running state is the fp32 recurrence of every token so far
    st = state.cpu().double().numpy()
    ref = np.stack([wk[:, Tt - 1], wv[:, Tt - 1]], axis=2)  # [B,H,2,d]
    err = np.abs(st - ref)
    assert (err <= 1e-3 * np.abs(ref) + 1e-5).all(), f"running state: max err {err.max():.3g}"


@pytest.mark.parametrize("mode,L", [(0, None), (0, 64), (0, 100)])
def test_scan_final_state(mode, L):
    """rat_scan_prefill's fp32 final state equals the oracle state at T-1
    (to fp32 rounding of a long recurrence)."""
    B, T, H, d = 2, 777, 3, 64
    x = inputs.make_random_prefill(B, T, H, d, torch.bfloat16, seed=11, gate_mean=2.0)
    fin = torch.full((B, H, 2, d), float("nan"), dtype=torch.float32, device="cuda")
    announce("scan final state", mode, L)
    rat.scan_prefill(x["k"].cuda(), x["v"].cuda(), x["gate"].cuda(), L=L, mode=mode, final_state=fin)
    torch.cuda.synchronize()
    wk, wv = oracle.scan(x["k"], x["v"], x["gate"], T if L is None else L, mode)
    ref = np.stack([wk[:, T - 1], wv[:, T - 1]], axis=2)
    got = fin.cpu().double().numpy()
    err = np.abs(got - ref)
    assert np.isfinite(got).all()
    assert (err <= FP32_RTOL * np.abs(ref) + FP32_ATOL).all(), f"max err {err.max():.3g}"


@pytest.mark.slow
def test_decode_step_full_size():
    """One decode-loop step on the 2.6B decode shape (B=64, T=32768, H=20,
    d=128, D=64, W=64) in the benchmark's launch configuration, with a state
    history that holds every position (n_cap = 32768 rows per head, more
    than 2^31 elements per cache).  Sampled heads are checked: the running
    state against the oracle's recurrence continued by one token, the written
    history row and ring slot, untouched neighbours, and the output against
    the oracle's decode over the residue's history rows and the ring."""
    w = inputs.DECODE_2P6B_D64
    B, T, H, d = w.B, w.T, w.H, w.d
    D, W = list(w.D), list(w.W)
    Dh, Wh = D[0], W[0]
    n_cap = Dh * ((T + Dh - 1) // Dh)
    p = T - 1
    P = 6  # prefix tokens whose recurrence gives the running state
    x = inputs.make_random_prefill(B, P + 1, H, d, torch.bfloat16, seed=21, gate_mean=1.5)
    wk, wv = oracle.scan(x["k"], x["v"], x["gate"], P + 1, 0)
    state = torch.from_numpy(np.stack([wk[:, P - 1], wv[:, P - 1]], axis=2)).float().cuda()  # [B,H,2,d]
    gen = torch.Generator(device="cuda")
    gen.manual_seed(22)
    mk = lambda *s: torch.randn(s, generator=gen, device="cuda").to(torch.bfloat16)  # noqa: E731
    q = mk(B, H, d)
    kc, vc = mk(B, H, n_cap, d), mk(B, H, n_cap, d)
    kw, vw = mk(B, H, Wh, d), mk(B, H, Wh, d)
    k_new, v_new, g_new = (x[n][:, P].contiguous().cuda() for n in ("k", "v", "gate"))
    mcap = n_cap // Dh
    r, j = p % Dh, p // Dh
    row = r * mcap + j  # the last row of the cache here (r = D - 1, j = mcap - 1)
    others = [row - 1, row - mcap, 0]  # same residue, same slot of another residue, first row
    samples = [(0, 0), (B - 1, H - 1), (17, 5), (40, 11), (63, 0)]
    before = {(b, h): (kc[b, h, others].cpu(), kw[b, h].cpu(), vw[b, h].cpu(),
                       kc[b, h, r * mcap:row].cpu(), vc[b, h, r * mcap:row].cpu())
              for b, h in samples}
    announce("decode step full size", w.name, "n_cap", n_cap)
    out = rat.decode_step(q, k_new, v_new, g_new, state, kc, vc, kw, vw, T, D, W)
    torch.cuda.synchronize()
    for b, h in samples:
        want_state = np.stack([wk[b, P, h], wv[b, P, h]])
        got_state = state[b, h].cpu().double().numpy()
        assert (np.abs(got_state - want_state) <= 1e-3 * np.abs(want_state) + 1e-5).all(), (b, h)
        other0, kw0, vw0, khist, vhist = before[(b, h)]
        # the new history row is the state rounded to bf16; its neighbours are untouched
        new_k = torch.from_numpy(want_state[0]).to(torch.bfloat16)
        assert (kc[b, h, row].cpu().float() - new_k.float()).abs().max() <= 2 ** -7 * new_k.float().abs().max()
        assert torch.equal(kc[b, h, others].cpu(), other0)
        # the ring holds the raw token in slot p mod W
        kw1 = kw0.clone()
        kw1[p % Wh] = x["k"][b, P, h]
        assert torch.equal(kw[b, h].cpu(), kw1)
        vw1 = vw0.clone()
        vw1[p % Wh] = x["v"][b, P, h]
        assert torch.equal(vw[b, h].cpu(), vw1)
        # output: the oracle's decode over this residue's rows 0 .. j (the
        # last one the oracle's new state in bf16) and the ring
        kd = torch.cat([khist, new_k[None]], 0)[None, None]
        vd = torch.cat([vhist, torch.from_numpy(want_state[1]).to(torch.bfloat16)[None]], 0)[None, None]
        want = oracle.attn_decode(q[b, h][None, None].cpu(), kd, vd, kw1[None, None], vw1[None, None], T,
                                  [Dh], [Wh], w.scale)
        assert_parity(out[b, h][None, None], want, torch.bfloat16, f"decode step b{b} h{h}")


@pytest.mark.parametrize("case", [
    # (B, T0, steps, H, d, D, W, L)
    (2, 300, 12, 3, 128, [1, 16, 64], [0, 8, 64], None),
    (1, 257, 10, 2, 64, [5, 1], [3, 0], 64),   # RESTART every 64 positions
])
def test_prefill_caches_then_decode(case):
    """The library builds the decode caches from its own prefill
    (build_decode_caches): the history rows and ring slots are exact copies
    of the states and raw tokens (rows and slots it must not write keep a
    sentinel), and a decode loop continued from them matches the oracle's
    prefill rows at the later positions."""
    B, T0, steps, H, d, D, W, L = case
    Tt = T0 + steps
    Lr = Tt if L is None else L
    x = inputs.make_random_prefill(B, Tt, H, d, torch.bfloat16, seed=12, gate_mean=1.5)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    pre = [t[:, :T0].contiguous() for t in (k, v, g)]
    state = torch.empty((B, H, 2, d), dtype=torch.float32, device="cuda")
    announce("prefill caches", case)
    ks, vs = rat.scan_prefill(*pre, L=min(Lr, T0), final_state=state)
    n_cap = rat.history_rows(Tt, D) + max(D)
    w_cap = max(W) + 2
    kc = torch.full((B, H, n_cap, d), 7.0, dtype=torch.bfloat16, device="cuda")
    vc = torch.full_like(kc, 7.0)
    kw = torch.full((B, H, w_cap, d), 7.0, dtype=torch.bfloat16, device="cuda")
    vw = torch.full_like(kw, 7.0)
    rat.build_decode_caches(ks, vs, pre[0], pre[1], D, W, n_cap=n_cap, w_cap=w_cap, kc=kc, vc=vc, kw=kw, vw=vw)
    torch.cuda.synchronize()
    kc_h, vc_h, kw_h, vw_h = kc.cpu(), vc.cpu(), kw.cpu(), vw.cpu()
    ks_h, vs_h = ks.cpu(), vs.cpu()
    for h, (Dh, Wh) in enumerate(zip(D, W)):
        p = np.arange(T0)
        rows = (p % Dh) * (n_cap // Dh) + p // Dh
        assert torch.equal(kc_h[:, h, rows], ks_h[:, :, h]) and torch.equal(vc_h[:, h, rows], vs_h[:, :, h]), h
        rest = np.setdiff1d(np.arange(n_cap), rows)
        assert (kc_h[:, h, rest] == 7.0).all() and (vc_h[:, h, rest] == 7.0).all(), h
        for s in range(w_cap):
            last = [t for t in range(max(0, T0 - Wh), T0) if Wh > 0 and t % Wh == s]
            if last:
                assert torch.equal(kw_h[:, h, s], x["k"][:, last[0], h]) and torch.equal(vw_h[:, h, s], x["v"][:, last[0], h])
            else:
                assert (kw_h[:, h, s] == 7.0).all() and (vw_h[:, h, s] == 7.0).all(), (h, s)
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
    assert_parity(torch.stack(got), want, torch.bfloat16, "decode after the library's caches")


# (B, T0, steps, H, d, D, W, L): decode loops continued from a SLIDING
# prefill (the recurrence window of the long workload, L = 64, and a general
# L), and from the first token
SLIDING_CASES = [
    (2, 100, 40, 2, 128, [64, 5], [128, 7], 64),
    (1, 0, 70, 2, 64, [16, 3], [16, 0], 64),
    (1, 300, 20, 3, 128, [64, 1, 9], [128, 0, 4], 33),
]
SLIDING_LOOP_CASES = [(c, torch.bfloat16) for c in SLIDING_CASES] + [(SLIDING_CASES[0], torch.float32),
                                                                       (SLIDING_CASES[2], torch.float32)]


def _sliding_loop(B, T0, steps, H, d, D, W, L, dtype, seed=5):
    """Prefill T0 tokens with the SLIDING window (states -> history, last L
    raw rows -> recurrence ring, last W -> attention ring), then decode
    `steps` tokens; returns (outputs [steps,B,H,d], oracle rows, kc, vc)."""
    Tt = T0 + steps
    x = inputs.make_random_prefill(B, Tt, H, d, dtype, seed=seed, gate_mean=1.0)
    q, k, v, g = (x[n].cuda() for n in ("q", "k", "v", "gate"))
    n_cap = max(Dh * ((Tt + Dh - 1) // Dh) for Dh in D) + 16
    w_cap = max(W) + 3
    if T0 > 0:
        pre = [t[:, :T0].contiguous() for t in (k, v, g)]
        ks, vs = rat.scan_prefill(*pre, L=L if L < T0 else T0, mode=rat.SLIDING)
        kc, vc = _history(ks, vs, T0, D, n_cap)
        rk, rv, rg = rat.sliding_state_from_prefill(*pre, L)
    else:
        kc = torch.zeros((B, H, n_cap, d), dtype=dtype, device="cuda")
        vc = torch.zeros_like(kc)
        rk = torch.zeros((B, H, L, d), dtype=dtype, device="cuda")
        rv, rg = torch.zeros_like(rk), torch.zeros_like(rk)
    kw, vw = _ring(k, v, T0, W, w_cap)
    got = []
    for T in range(T0 + 1, Tt + 1):
        t = T - 1
        out = rat.decode_step_sliding(q[:, t].contiguous(), k[:, t].contiguous(), v[:, t].contiguous(),
                                      g[:, t].contiguous(), rk, rv, rg, kc, vc, kw, vw, T, D, W)
        got.append(out.clone())
    torch.cuda.synchronize()
    wk, wv = oracle.scan(x["k"], x["v"], x["gate"], L, oracle.MODE_SLIDING)
    rows = np.array([(b, t, h) for t in range(T0, Tt) for b in range(B) for h in range(H)], np.int32)
    want = oracle.attn_prefill_rows(x["q"], wk, wv, x["k"], x["v"], rows, D, W, 1 / math.sqrt(d))
    return torch.stack(got), want.reshape(steps, B, H, d), (kc, vc, wk, wv, n_cap)


@pytest.mark.parametrize("case,dtype", SLIDING_LOOP_CASES,
                         ids=lambda c: f"B{c[0]}T{c[1]}+{c[2]}H{c[3]}d{c[4]}D{c[5]}W{c[6]}L{c[7]}"
                         if isinstance(c, tuple) else str(c)[6:])
def test_decode_loop_sliding(case, dtype):
    """Every step's output equals the oracle's prefill output at that
    position with the SLIDING states (explicit window sums), and the states
    the loop appended to the history equal the oracle's."""
    B, T0, steps, H, d, D, W, L = case
    announce("sliding decode loop", case, dtype)
    got, want, (kc, vc, wk, wv, n_cap) = _sliding_loop(B, T0, steps, H, d, D, W, L, dtype)
    assert_parity(got, want, dtype, "sliding decode loop outputs")
    kc_h, vc_h = kc.cpu(), vc.cpu()
    for h, Dh in enumerate(D):
        p = np.arange(T0, T0 + steps)
        hr = (p % Dh) * (n_cap // Dh) + p // Dh
        assert_parity(kc_h[:, h, hr], wk[:, T0:T0 + steps, h], dtype, f"k history head {h}")
        assert_parity(vc_h[:, h, hr], wv[:, T0:T0 + steps, h], dtype, f"v history head {h}")


def test_sliding_state_from_prefill_exact():
    """The recurrence ring of a prefill holds the raw rows of its last L
    positions bit for bit in slots p mod L; slots with no position (T < L)
    keep their contents."""
    for (B, T, H, d, L) in ((2, 150, 3, 128, 64), (1, 40, 2, 64, 64), (1, 64, 1, 128, 64), (2, 77, 2, 64, 10)):
        x = inputs.make_random_prefill(B, T, H, d, torch.bfloat16, seed=9)
        k, v, g = (x[n].cuda() for n in ("k", "v", "gate"))
        sentinel = 7.0
        rk = torch.full((B, H, L, d), sentinel, dtype=torch.bfloat16, device="cuda")
        rv, rg = torch.full_like(rk, sentinel), torch.full_like(rk, sentinel)
        announce("sliding state fill", (B, T, H, d, L))
        rat.sliding_state_from_prefill(k, v, g, L, rk=rk, rv=rv, rg=rg)
        torch.cuda.synchronize()
        for name, ring, src in (("k", rk, x["k"]), ("v", rv, x["v"]), ("g", rg, x["gate"])):
            ring = ring.cpu()
            for slot in range(L):
                p = (T - 1) - ((T - 1 - slot) % L)
                if p >= 0:
                    assert torch.equal(ring[:, :, slot], src[:, p]), (name, slot, p)
                else:
                    assert (ring[:, :, slot] == sentinel).all(), (name, slot)


@pytest.mark.slow
def test_decode_loop_sliding_long_workload():
    """A decode loop continued from a prefill of the 16K windowed workload's
    shape (H=16, d=128, D=64, W=128, SLIDING L=64, gate logits ~ N(1,1))."""
    w = inputs.PREFILL_LONG
    B, steps = 1, 6
    T0 = w.T - steps
    announce("sliding decode loop, long workload shape")
    got, want, _ = _sliding_loop(B, T0, steps, w.H, w.d, list(w.D), list(w.W), w.L, w.dtype, seed=12)
    assert_parity(got, want, w.dtype, "sliding decode after the long prefill")
