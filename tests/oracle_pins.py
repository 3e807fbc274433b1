"""Pins of the CPU oracle: checks against what the pages and the mathematics
fix, written so that each takes an ``oracle.oracle.Oracle`` instance.

``test_oracle_pins.py`` runs them on the oracle itself; ``test_oracle_mutants.py``
runs them on deliberately broken copies of ``oracle.c`` to show that every
planted mistake is caught by at least one pin.

Sources: "RAT+ Deep Dive" (zhichai.net) S1 (tokens skip a fixed interval D),
S2.1 (forget-gate recurrence, 64-token window, L = T, parallel prefill by an
associative scan), S3.1 table (attention FLOPs T/D), S6 Head-Wise Hybrid;
the RAT+ abstract (arXiv 2602.18196: FLOPs and KV cache fall by D, 64x at
D = 64; dilated attention optionally with local windows).
"""
from __future__ import annotations

import math
import os

import numpy as np
import torch

from oracle import brute

GOLDEN = os.path.join(os.path.dirname(os.path.abspath(__file__)), "golden")


def _rng(seed):
    return np.random.default_rng(seed)


def _inputs(seed, B, T, H, d, gate_mean=1.0):
    r = _rng(seed)
    q = r.standard_normal((B, T, H, d))
    k = r.standard_normal((B, T, H, d))
    v = r.standard_normal((B, T, H, d))
    lg = r.standard_normal((B, T, H, d)) + gate_mean
    return q, k, v, lg


def read_golden(name):
    rows = []
    with open(os.path.join(GOLDEN, name)) as f:
        for line in f:
            line = line.split("#", 1)[0].strip()
            if line:
                rows.append([int(x) for x in line.split()])
    return rows


# ---------------------------------------------------------------- gates
def pin_gate_values(o):
    """sigmoid pairs: limits, the midpoint and scipy's logistic function."""
    from scipy.special import expit

    x = np.array([-np.inf, -30.0, -1.5, 0.0, 0.25, 3.0, 40.0, np.inf])
    g, gb = o.gates(x)
    assert g[0] == 0.0 and gb[0] == 1.0  # l = -inf: forget everything
    assert g[-1] == 1.0 and gb[-1] == 0.0  # l = +inf: keep everything
    assert g[3] == 0.5 and gb[3] == 0.5
    np.testing.assert_allclose(g, expit(x), rtol=1e-15, atol=0)
    np.testing.assert_allclose(gb, expit(-x), rtol=1e-15, atol=0)


# ---------------------------------------------------------------- scan
def pin_scan_hand_example(o):
    """T = 3, one channel, logit 0 (g = 1/2), x = 1, 2, 3, worked by hand:
    full: h = 1/2, 1/4 + 1 = 5/4, 5/8 + 3/2 = 17/8;
    RESTART, L = 2: the block starting at t = 2 gives h_2 = 3/2;
    SLIDING, L = 2: h_2 = g_2 (1-g_1) x_1 + (1-g_2) x_2 = 1/2 + 3/2 = 2.
    The values are dyadic, hence exact in fp64."""
    x = np.array([1.0, 2.0, 3.0]).reshape(1, 3, 1, 1)
    lg = np.zeros_like(x)
    ks, vs = o.scan(x, 2 * x, lg, L=3)
    assert ks.ravel().tolist() == [0.5, 1.25, 2.125]
    assert vs.ravel().tolist() == [1.0, 2.5, 4.25]
    ks, _ = o.scan(x, x, lg, L=2, mode=0)
    assert ks.ravel().tolist() == [0.5, 1.25, 1.5]
    ks, _ = o.scan(x, x, lg, L=2, mode=1)
    assert ks.ravel().tolist() == [0.5, 1.25, 2.0]


def pin_scan_constant_closed_form(o):
    """Constant gate g and constant input x: h_t = x (1 - g^n_t) with
    n_t = t+1 (full), (t mod L)+1 (RESTART), min(t+1, L) (SLIDING)."""
    T, L, xval = 50, 7, 1.75
    g = 0.75
    lg = np.full((1, T, 1, 1), math.log(g / (1 - g)))
    x = np.full((1, T, 1, 1), xval)
    t = np.arange(T)
    for mode, n in ((None, t + 1), (0, t % L + 1), (1, np.minimum(t + 1, L))):
        if mode is None:
            ks, _ = o.scan(x, x, lg, L=T)
        else:
            ks, _ = o.scan(x, x, lg, L=L, mode=mode)
        np.testing.assert_allclose(ks.ravel(), xval * (1 - g ** n), rtol=1e-13, atol=0)


def pin_scan_special_cases(o):
    q, k, v, lg = _inputs(1, 2, 40, 2, 3)
    # g = 0 (logit -inf): the state is the input itself, exactly
    ks, vs = o.scan(k, v, np.full_like(lg, -np.inf), L=40)
    assert np.array_equal(ks, k) and np.array_equal(vs, v)
    # g = 1 (logit +inf): nothing ever enters the state
    ks, vs = o.scan(k, v, np.full_like(lg, np.inf), L=40)
    assert np.all(ks == 0) and np.all(vs == 0)
    # L = 1: h = (1-g) x in both windowed modes
    _, gb = o.gates(lg)
    for mode in (0, 1):
        ks, vs = o.scan(k, v, lg, L=1, mode=mode)
        np.testing.assert_allclose(ks, gb * k, rtol=1e-15, atol=0)
        np.testing.assert_allclose(vs, gb * v, rtol=1e-15, atol=0)
    # L >= T: both windowed modes are the full recurrence
    full = o.scan(k, v, lg, L=40)
    for mode in (0, 1):
        for L in (40, 41, 1000):
            got = o.scan(k, v, lg, L=L, mode=mode)
            assert np.array_equal(got[0], full[0]) and np.array_equal(got[1], full[1])


def pin_scan_explicit_sum(o):
    """Brute force on tiny T: the closed double sum of every mode."""
    q, k, v, lg = _inputs(2, 2, 37, 2, 3, gate_mean=0.5)
    for L, mode in ((37, 0), (8, 0), (8, 1), (5, 1), (1, 0), (64, 1)):
        want = brute.scan_explicit(k, v, lg, L, mode)
        got = o.scan(k, v, lg, L=L, mode=mode)
        np.testing.assert_allclose(got[0], want[0], rtol=1e-12, atol=1e-14)
        np.testing.assert_allclose(got[1], want[1], rtol=1e-12, atol=1e-14)


def pin_scan_parallel_prefix(o):
    """Sequential recurrence == log-depth associative scan (full and RESTART)."""
    q, k, v, lg = _inputs(3, 2, 200, 2, 4, gate_mean=2.0)
    for L in (200, 64, 13):
        want = brute.scan_parallel(k, v, lg, L)
        got = o.scan(k, v, lg, L=L, mode=0)
        np.testing.assert_allclose(got[0], want[0], rtol=1e-11, atol=1e-13)
        np.testing.assert_allclose(got[1], want[1], rtol=1e-11, atol=1e-13)


# ---------------------------------------------------------------- index sets
def pin_index_sets_by_hand(o):
    dil, loc = o.index_sets(10, 4, 3)
    assert dil.tolist() == [10, 6, 2] and loc.tolist() == [10, 9, 8]
    dil, loc = o.index_sets(1, 4, 3)
    assert dil.tolist() == [1] and loc.tolist() == [1, 0]
    dil, loc = o.index_sets(0, 1, 0)
    assert dil.tolist() == [0] and loc.tolist() == []
    dil, loc = o.index_sets(7, 1, 2)
    assert dil.tolist() == [7, 6, 5, 4, 3, 2, 1, 0] and loc.tolist() == [7, 6]
    dil, loc = o.index_sets(63, 64, 64)
    assert dil.tolist() == [63] and loc.tolist() == list(range(63, -1, -1))


def pin_pair_counts_closed_form(o):
    """sum_t |S_dil(t)| = sum_r M_r (M_r+1)/2 with M_r = ceil((T-r)/D)
    (= D M (M+1)/2 when D divides T); sum_t |S_loc(t)| = W(W+1)/2 + (T-W) W
    for T >= W, T(T+1)/2 otherwise."""
    for T, D, W in ((256, 4, 0), (4096, 16, 0), (16384, 64, 128), (100, 7, 13),
                    (37, 64, 5), (10, 3, 50), (32768, 1, 0), (300, 300, 1)):
        nd, nl = o.count_pairs(T, D, W)
        want_d = sum(((T - r + D - 1) // D) * ((T - r + D - 1) // D + 1) // 2
                     for r in range(min(D, T)))
        if T % D == 0:
            M = T // D
            assert want_d == D * M * (M + 1) // 2
        want_l = W * (W + 1) // 2 + (T - W) * W if T >= W else T * (T + 1) // 2
        assert (nd, nl) == (want_d, want_l), (T, D, W)


def pin_pages_flops_table(o):
    """Deep Dive S3.1 table: a query's attention FLOPs are T/D; the RAT+
    abstract: the KV cache and FLOPs fall by exactly D (64x at D = 64)."""
    T = 4096
    for D, divisor in read_golden("flops_per_query_vs_dilation.txt"):
        dil, loc = o.index_sets(T - 1, D, 0)
        assert len(loc) == 0
        assert len(dil) * divisor == T  # keys of the last query: T / D
        assert len(dil) == (T - 1) // D + 1  # = the decode cache entries
    for D, factor in read_golden("kv_cache_reduction.txt"):
        dense, _ = o.index_sets(T - 1, 1, 0)
        dil, _ = o.index_sets(T - 1, D, 0)
        assert len(dense) == factor * len(dil)


# ---------------------------------------------------------------- attention
def _sdpa_causal(q, k, v, scale):
    """torch's scaled_dot_product_attention on the CPU in fp64; [n, d] rows."""
    qt = torch.from_numpy(q)[None, None]
    kt = torch.from_numpy(k)[None, None]
    vt = torch.from_numpy(v)[None, None]
    out = torch.nn.functional.scaled_dot_product_attention(qt, kt, vt, is_causal=True,
                                                           scale=scale)
    return out[0, 0].numpy()


def pin_attn_dense_is_sdpa(o):
    """g = 0 (states = raw inputs), D = 1, W = 0: dense causal softmax
    attention, i.e. the library routine."""
    q, k, v, lg = _inputs(4, 2, 45, 3, 8)
    ks, vs = o.scan(k, v, np.full_like(lg, -np.inf), L=45)
    scale = 1 / math.sqrt(8)
    out = o.attn_prefill(q, ks, vs, None, None, 1, 0, scale)
    for b in range(2):
        for h in range(3):
            want = _sdpa_causal(q[b, :, h], k[b, :, h], v[b, :, h], scale)
            np.testing.assert_allclose(out[b, :, h], want, rtol=1e-12, atol=1e-13)


def pin_attn_residue_decomposition(o):
    """W = 0: the rows of residue r are causal attention over q[r::D],
    states[r::D] (ragged T, several D)."""
    q, ks, vs, _ = _inputs(5, 1, 53, 2, 8)
    scale = 0.3
    for D in (2, 4, 7, 16):
        out = o.attn_prefill(q, ks, vs, None, None, D, 0, scale)
        for h in range(2):
            for r in range(D):
                want = _sdpa_causal(q[0, r::D, h], ks[0, r::D, h], vs[0, r::D, h], scale)
                np.testing.assert_allclose(out[0, r::D, h], want, rtol=1e-12, atol=1e-13)


def pin_attn_single_key(o):
    """D >= T, W = 0: one key per query, the output IS that state's value."""
    q, ks, vs, _ = _inputs(6, 2, 20, 2, 8)
    for D in (20, 21, 1000):
        out = o.attn_prefill(q, ks, vs, None, None, D, 0, 0.5)
        assert np.array_equal(out, vs)


def pin_attn_two_key_closed_form(o):
    """D >= T, W = 1: keys {state_t, raw_t}; the softmax of two logits a, b
    gives sigmoid(a-b) * Vstate + sigmoid(b-a) * vraw."""
    from scipy.special import expit

    q, ks, vs, _ = _inputs(7, 1, 30, 2, 8)
    _, kr, vr, _ = _inputs(8, 1, 30, 2, 8)
    scale = 0.4
    out = o.attn_prefill(q, ks, vs, kr, vr, 64, 1, scale)
    a = scale * np.sum(q * ks, axis=-1, keepdims=True)
    b = scale * np.sum(q * kr, axis=-1, keepdims=True)
    want = expit(a - b) * vs + expit(b - a) * vr
    np.testing.assert_allclose(out, want, rtol=1e-12, atol=1e-13)


def pin_attn_masked_matrix(o):
    """Brute force on tiny T: the dense masked-score formulation over
    [states ; raw] for mixed per-head (D, W)."""
    q, ks, vs, _ = _inputs(9, 2, 70, 5, 8)
    _, kr, vr, _ = _inputs(10, 2, 70, 5, 8)
    D = [1, 3, 8, 64, 5]
    W = [0, 4, 16, 9, 70]
    out = o.attn_prefill(q, ks, vs, kr, vr, D, W, 0.35)
    want = brute.attn_masked(q, ks, vs, kr, vr, D, W, 0.35)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-12)


def pin_attn_hybrid_heads(o):
    """Head-wise hybrid (Deep Dive S6): each head of a mixed run equals the
    run of that head alone."""
    q, ks, vs, _ = _inputs(11, 1, 64, 4, 8)
    _, kr, vr, _ = _inputs(12, 1, 64, 4, 8)
    D = [1, 1, 4, 16]
    W = [0, 0, 8, 32]
    out = o.attn_prefill(q, ks, vs, kr, vr, D, W, 0.3)
    for h in range(4):
        one = o.attn_prefill(q[:, :, h:h + 1], ks[:, :, h:h + 1], vs[:, :, h:h + 1],
                             kr[:, :, h:h + 1], vr[:, :, h:h + 1], D[h], W[h], 0.3)
        assert np.array_equal(out[:, :, h:h + 1], one)


def pin_rows_match_full(o):
    q, ks, vs, _ = _inputs(13, 2, 50, 3, 8)
    _, kr, vr, _ = _inputs(14, 2, 50, 3, 8)
    D, W = [1, 4, 9], [0, 6, 12]
    full = o.attn_prefill(q, ks, vs, kr, vr, D, W, 0.3)
    rows = [(0, 0, 0), (1, 49, 2), (0, 17, 1), (1, 8, 2)]
    got = o.attn_prefill_rows(q, ks, vs, kr, vr, rows, D, W, 0.3)
    for i, (b, t, h) in enumerate(rows):
        assert np.array_equal(got[i], full[b, t, h])


# ---------------------------------------------------------------- decode
def decode_caches_from_prefill(ks, vs, k, v, T, D, W, nd_cap, w_cap, rng):
    """Lay prefill states / raw tokens out as decode caches at context T:
    dilated entry i = state at position ((T-1) mod D) + i D, ring = the
    last min(W, T) raw tokens in a shuffled slot order."""
    B, _, H, d = ks.shape
    kd = np.zeros((B, H, nd_cap, d))
    vd = np.zeros((B, H, nd_cap, d))
    kw = np.zeros((B, H, w_cap, d))
    vw = np.zeros((B, H, w_cap, d))
    for h in range(H):
        r = (T - 1) % D[h]
        pos = np.arange(r, T, D[h])
        kd[:, h, : len(pos)] = ks[:, pos, h]
        vd[:, h, : len(pos)] = vs[:, pos, h]
        nw = min(W[h], T)
        wpos = np.arange(T - nw, T)
        rng.shuffle(wpos)
        kw[:, h, :nw] = k[:, wpos, h]
        vw[:, h, :nw] = v[:, wpos, h]
    return kd, vd, kw, vw


def pin_decode_equals_prefill_row(o):
    """Decode at context T equals prefill row T-1 (two separate code paths)."""
    q, k, v, lg = _inputs(15, 2, 77, 4, 8)
    D, W = [1, 4, 16, 100], [0, 8, 5, 3]
    ks, vs = o.scan(k, v, lg, L=77)
    pre = o.attn_prefill(q, ks, vs, k, v, D, W, 0.3)
    rng = _rng(0)
    for T in (1, 2, 33, 77):
        nd_cap = max((T + Dh - 1) // Dh for Dh in D) + 3
        w_cap = max(min(Wh, T) for Wh in W) + 2
        kd, vd, kw, vw = decode_caches_from_prefill(ks[:, :T], vs[:, :T], k[:, :T], v[:, :T],
                                                    T, D, W, nd_cap, w_cap, rng)
        pre_T = o.attn_prefill(q[:, :T], ks[:, :T], vs[:, :T], k[:, :T], v[:, :T], D, W, 0.3)
        got = o.attn_decode(q[:, T - 1], kd, vd, kw, vw, T, D, W, 0.3)
        np.testing.assert_allclose(got, pre_T[:, T - 1], rtol=1e-12, atol=1e-13)
        if T == 77:
            np.testing.assert_allclose(got, pre[:, T - 1], rtol=1e-12, atol=1e-13)


def pin_decode_ring_order(o):
    """Ring slot order does not matter (a softmax is permutation invariant)."""
    r = _rng(16)
    B, H, d, T = 2, 3, 8, 500
    D, W = [16, 64, 7], [10, 33, 1]
    nd_cap, w_cap = 80, 40
    q = r.standard_normal((B, H, d))
    kd, vd = r.standard_normal((2, B, H, nd_cap, d))
    kw, vw = r.standard_normal((2, B, H, w_cap, d))
    base = o.attn_decode(q, kd, vd, kw, vw, T, D, W, 0.3)
    perm = r.permutation(10)  # permute only the valid slots of head 0
    kw2, vw2 = kw.copy(), vw.copy()
    kw2[:, 0, :10] = kw[:, 0, perm]
    vw2[:, 0, :10] = vw[:, 0, perm]
    got = o.attn_decode(q, kd, vd, kw2, vw2, T, D, W, 0.3)
    np.testing.assert_allclose(got, base, rtol=1e-13, atol=1e-14)
    # entries past the valid counts are never read
    kd3, kw3 = kd.copy(), kw.copy()
    for h in range(H):
        kd3[:, h, (T + D[h] - 1) // D[h]:] = np.nan  # entries past ceil(T/D)
        kw3[:, h, min(W[h], T):] = np.nan  # slots past min(W, T)
    got = o.attn_decode(q, kd3, vd, kw3, vw, T, D, W, 0.3)
    np.testing.assert_array_equal(got, base)


# ---------------------------------------------------------------- chunk grid
# The absolute reading of the dilated pattern, after the RAT page ("RAT:
# Bridging RNN Efficiency and Attention Accuracy via Chunk-based Sequence
# Modeling", Abstract: chunks, attention across chunks): query t sees the
# states ending a chunk of D tokens before t, and its own state.
def pin_chunk_index_sets_by_hand(o):
    assert o.chunk_index_set(9, 4).tolist() == [3, 7, 9]
    assert o.chunk_index_set(3, 4).tolist() == [3]       # its own state ends the chunk
    assert o.chunk_index_set(4, 4).tolist() == [3, 4]
    assert o.chunk_index_set(0, 1).tolist() == [0]
    assert o.chunk_index_set(5, 1).tolist() == [0, 1, 2, 3, 4, 5]
    for D in (1, 2, 3, 16, 64):
        for t in range(0, 200, 7):
            got = o.chunk_index_set(t, D).tolist()
            want = sorted({p for p in range(t) if p % D == D - 1} | {t})
            assert got == want, (t, D)
            assert len(got) == t // D + 1  # as many keys as the relative reading


def pin_chunk_attn_dense_is_sdpa(o):
    """D = 1: every earlier position ends a chunk -- dense causal attention."""
    q, ks, vs, _ = _inputs(21, 2, 41, 2, 8)
    scale = 1 / math.sqrt(8)
    out = o.chunk_attn_prefill(q, ks, vs, 1, scale)
    for b in range(2):
        for h in range(2):
            want = _sdpa_causal(q[b, :, h], ks[b, :, h], vs[b, :, h], scale)
            np.testing.assert_allclose(out[b, :, h], want, rtol=1e-12, atol=1e-13)


def pin_chunk_attn_chunk_ends(o):
    """Queries that end a chunk (t mod D = D - 1) see exactly the chunk ends
    up to t: causal attention over q[D-1::D], states[D-1::D]."""
    q, ks, vs, _ = _inputs(22, 1, 61, 2, 8)
    for D in (2, 5, 16):
        out = o.chunk_attn_prefill(q, ks, vs, D, 0.3)
        for h in range(2):
            want = _sdpa_causal(q[0, D - 1::D, h], ks[0, D - 1::D, h], vs[0, D - 1::D, h], 0.3)
            np.testing.assert_allclose(out[0, D - 1::D, h], want, rtol=1e-12, atol=1e-13)


def pin_chunk_attn_own_state_only(o):
    """Before the first chunk end (t < D) a query has one key, its own
    state: the output IS that state's value."""
    q, ks, vs, _ = _inputs(23, 2, 30, 2, 8)
    for D in (8, 30, 1000):
        out = o.chunk_attn_prefill(q, ks, vs, D, 0.5)
        n = min(D, 30)
        assert np.array_equal(out[:, :n], vs[:, :n])


def pin_chunk_attn_masked_matrix(o):
    """Brute force on tiny T: one dense masked softmax per head (mixed D)."""
    q, ks, vs, _ = _inputs(24, 2, 67, 4, 8)
    D = [1, 3, 8, 20]
    out = o.chunk_attn_prefill(q, ks, vs, D, 0.35)
    want = brute.chunk_attn_masked(q, ks, vs, D, 0.35)
    np.testing.assert_allclose(out, want, rtol=1e-11, atol=1e-12)


# ---------------------------------------------------------------- backward
def _layer_loss(o, q, k, v, lg, dout, L, mode, D, W, scale):
    """<dout, out> of the oracle's forward (recurrence, then attention)."""
    ks, vs = o.scan(k, v, lg, L, mode)
    need_raw = any(w > 0 for w in W)
    out = o.attn_prefill(q, ks, vs, k if need_raw else None, v if need_raw else None, D, W, scale)
    return float(np.sum(dout * out))


def pin_backward_finite_differences(o):
    """The backward against central differences of the (separately pinned)
    forward, element by element, for the full recurrence, RESTART and a
    SLIDING window, dense, dilated and windowed heads together: every input
    of every tensor."""
    eps = 1e-5
    for (T, L, mode, D, W) in [(10, 10, 0, [1, 3], [0, 2]), (11, 4, 0, [2, 1], [3, 0]), (9, 9, 0, [4, 20], [1, 0]),
                               (12, 4, 1, [1, 3], [0, 2]), (10, 3, 1, [2, 1], [3, 0]), (8, 5, 1, [1, 20], [0, 1])]:
        q, k, v, lg = _inputs(40 + T + 7 * mode, 1, T, 2, 3, gate_mean=0.5)
        dout = _rng(41 + T + 7 * mode).standard_normal(q.shape)
        args = (L, mode, D, W, 0.7)
        grads = o.layer_backward(q, k, v, lg, dout, *args)
        for which, (x, g) in enumerate(zip((q, k, v, lg), grads)):
            fd = np.empty_like(x)
            for idx in np.ndindex(x.shape):
                saved = x[idx]
                x[idx] = saved + eps
                up = _layer_loss(o, q, k, v, lg, dout, *args)
                x[idx] = saved - eps
                dn = _layer_loss(o, q, k, v, lg, dout, *args)
                x[idx] = saved
                fd[idx] = (up - dn) / (2 * eps)
            np.testing.assert_allclose(g, fd, rtol=1e-6, atol=1e-8, err_msg=f"input {which} T={T} L={L} mode={mode}")


def pin_backward_own_state_only(o):
    """D >= T and no window: each query's only key is its own state, so
    out_t = v_state_t, dq = 0, the keys get no gradient, and the value
    gradient is the reverse recurrence of dout: with a constant gate g,
    dL/dv_state_t = sum_{s >= t} g^(s-t) dout_s and dv_t = (1 - g) times it."""
    B, T, H, d = 2, 12, 2, 5
    q, k, v, _ = _inputs(45, B, T, H, d)
    lg = np.full(q.shape, 0.8)
    dout = _rng(46).standard_normal(q.shape)
    dq, dk, dv, dl = o.layer_backward(q, k, v, lg, dout, T, 0, [T, 50], [0, 0], 0.5)
    assert np.array_equal(dq, np.zeros_like(dq))
    assert np.array_equal(dk, np.zeros_like(dk))
    g = 1.0 / (1.0 + math.exp(-0.8))
    lam = np.zeros_like(dout)
    for t in range(T):
        for s in range(t, T):
            lam[:, t] += g ** (s - t) * dout[:, s]
    np.testing.assert_allclose(dv, (1 - g) * lam, rtol=1e-12, atol=1e-14)
    _, vs = o.scan(k, v, lg, T, 0)
    prev = np.concatenate([np.zeros_like(vs[:, :1]), vs[:, :-1]], axis=1)
    np.testing.assert_allclose(dl, g * (1 - g) * lam * (prev - v), rtol=1e-11, atol=1e-13)


def pin_backward_sliding_one_token(o):
    """SLIDING at L = 1: each state is (1 - g_t) x_t alone, so with
    lambda = dLoss/dstate (from the attention) dx_t = (1 - g_t) lambda_t and
    dlogit_t = -g_t (1 - g_t) sum_{x in k, v} lambda_t x_t.  With D >= T, no
    window and a zero query, each query's only key is its own state with
    weight one, so lambda_v = dout and lambda_k = 0."""
    B, T, H, d = 1, 9, 2, 4
    _, k, v, lg = _inputs(47, B, T, H, d)
    q = np.zeros_like(k)
    dout = _rng(48).standard_normal(q.shape)
    dq, dk, dv, dl = o.layer_backward(q, k, v, lg, dout, 1, 1, [T, T], [0, 0], 0.9)
    g = 1.0 / (1.0 + np.exp(-lg))
    np.testing.assert_allclose(dv, (1 - g) * dout, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dk, np.zeros_like(dk), atol=1e-14)
    np.testing.assert_allclose(dl, -g * (1 - g) * dout * v, rtol=1e-11, atol=1e-14)


def pin_backward_states_at_scan_states(o):
    """The backward at given states, handed the recurrence's own states, is
    the layer backward (which the finite differences above pin): full,
    RESTART and SLIDING."""
    for (T, L, mode) in [(11, 11, 0), (11, 4, 0), (10, 3, 1)]:
        q, k, v, lg = _inputs(50 + T + L, 2, T, 2, 3)
        dout = _rng(51 + T).standard_normal(q.shape)
        args = (L, mode, [1, 3], [0, 2], 0.6)
        ks, vs = o.scan(k, v, lg, L, mode)
        want = o.layer_backward(q, k, v, lg, dout, *args)
        got = o.layer_backward_states(q, k, v, lg, ks, vs, dout, *args)
        for g, w in zip(got, want):
            assert np.array_equal(g, w)


def pin_backward_states_dq_finite_differences(o):
    """At states that no recurrence produced (random ones), dq is still the
    gradient of <dout, attention(q, states, raw window)> in q with the states
    held fixed: central differences of the forward attention, every element,
    with dense, dilated and windowed heads."""
    eps = 1e-5
    B, T, H, d = 1, 10, 3, 3
    q, k, v, lg = _inputs(52, B, T, H, d)
    r = _rng(53)
    ks, vs = r.standard_normal(q.shape), r.standard_normal(q.shape)
    dout = r.standard_normal(q.shape)
    D, W, scale = [1, 3, 20], [0, 2, 4], 0.8
    dq = o.layer_backward_states(q, k, v, lg, ks, vs, dout, T, 0, D, W, scale)[0]
    loss = lambda: float(np.sum(dout * o.attn_prefill(q, ks, vs, k, v, D, W, scale)))
    fd = np.empty_like(q)
    for idx in np.ndindex(q.shape):
        saved = q[idx]
        q[idx] = saved + eps
        up = loss()
        q[idx] = saved - eps
        dn = loss()
        q[idx] = saved
        fd[idx] = (up - dn) / (2 * eps)
    np.testing.assert_allclose(dq, fd, rtol=1e-6, atol=1e-8)


def pin_backward_states_gate_term(o):
    """The given states enter the recurrence's backward through h_{t-1} in the
    gate derivative.  With D >= T, no window and a zero query, each query's
    only key is its own state with weight one, whatever the states are: so
    lambda_v is the reverse recurrence of dout, lambda_k = 0, dk = 0, dv =
    (1 - g) lambda_v and dlogit_t = g (1 - g) lambda_v,t (vs_{t-1} - v_t) with
    vs the given (random) value states."""
    B, T, H, d = 2, 9, 2, 4
    _, k, v, _ = _inputs(54, B, T, H, d)
    q = np.zeros_like(k)
    lg = np.full(q.shape, 0.4)
    r = _rng(55)
    ks, vs = r.standard_normal(q.shape), r.standard_normal(q.shape)
    dout = r.standard_normal(q.shape)
    dq, dk, dv, dl = o.layer_backward_states(q, k, v, lg, ks, vs, dout, T, 0, [T, 40], [0, 0], 0.5)
    g = 1.0 / (1.0 + math.exp(-0.4))
    lam = np.zeros_like(dout)
    for t in range(T):
        for s_ in range(t, T):
            lam[:, t] += g ** (s_ - t) * dout[:, s_]
    prev = np.concatenate([np.zeros_like(vs[:, :1]), vs[:, :-1]], axis=1)
    assert np.array_equal(dq, np.zeros_like(dq))
    assert np.array_equal(dk, np.zeros_like(dk))
    np.testing.assert_allclose(dv, (1 - g) * lam, rtol=1e-12, atol=1e-14)
    np.testing.assert_allclose(dl, g * (1 - g) * lam * (prev - v), rtol=1e-11, atol=1e-13)


ALL_PINS = [v for k, v in sorted(globals().items()) if k.startswith("pin_")]
