"""Second, independent fp64 formulations used to pin the C oracle on tiny inputs.

TEST INFRASTRUCTURE ONLY (imported by ``tests/`` alone).

Each function computes the same quantity as ``oracle.c`` by a different route,
so that a dropped term, a wrong sign or index, or a transposed operand in
either one shows up as a disagreement:

* ``scan_explicit`` -- the recurrence of "RAT+ Deep Dive" S2.1 written out as
  its closed double sum h_t = sum_s (prod_{r=s+1}^t g_r) (1-g_s) x_s over the
  window of t (whole prefix, the RESTART block of t, or the last L tokens).
* ``scan_parallel`` -- the same recurrence as a Hillis-Steele parallel prefix
  over the associative pairs (a, b) with (a1,b1)+(a2,b2) = (a1 a2, a2 b1 + b2)
  (the "parallel prefill via associative scan" of Deep Dive S2.1 / S7.3).
* ``attn_masked`` -- dilated + local attention (Deep Dive S1; RAT+ abstract)
  as ONE dense score matrix over the concatenated key set [states ; raw keys]
  with a boolean mask, softmax by numpy over the key axis.

Pure Python / numpy, meant for T of at most a few hundred.
"""
from __future__ import annotations

import numpy as np


def _sig(x):
    x = np.asarray(x, dtype=np.float64)
    with np.errstate(over="ignore"):
        return 1.0 / (1.0 + np.exp(-x)), 1.0 / (1.0 + np.exp(x))


def window_start(t, T, L, mode):
    """First position summed into h_t."""
    if L >= T:
        return 0
    if mode == 0:  # RESTART: the block of length L that holds t
        return (t // L) * L
    return max(0, t - L + 1)  # SLIDING: last L tokens


def scan_explicit(k, v, logit, L, mode):
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g, gb = _sig(logit)
    B, T, H, d = k.shape
    ks = np.zeros_like(k)
    vs = np.zeros_like(v)
    for t in range(T):
        lo = window_start(t, T, L, mode)
        for s in range(lo, t + 1):
            w = gb[:, s] * np.prod(g[:, s + 1:t + 1], axis=1)  # [B,H,d]
            ks[:, t] += w * k[:, s]
            vs[:, t] += w * v[:, s]
    return ks, vs


def scan_parallel(k, v, logit, L):
    """Full (L >= T) or RESTART scan by a log-depth associative prefix."""
    k = np.asarray(k, np.float64)
    v = np.asarray(v, np.float64)
    g, gb = _sig(logit)
    B, T, H, d = k.shape
    a = g.copy()
    if L < T:
        a[:, ::L] = 0.0  # a block start forgets everything before it
    bk = gb * k
    bv = gb * v
    off = 1
    while off < T:
        a_prev, bk_prev, bv_prev = a[:, :-off].copy(), bk[:, :-off].copy(), bv[:, :-off].copy()
        # element t combines with element t-off (the earlier one on the left)
        bk[:, off:] = a[:, off:] * bk_prev + bk[:, off:]
        bv[:, off:] = a[:, off:] * bv_prev + bv[:, off:]
        a[:, off:] = a_prev * a[:, off:]
        off *= 2
    return bk, bv


def attention_mask(T, D, W):
    """Boolean [T, 2T] mask over [states ; raw]: key s (state) or T+u (raw)."""
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    dil = (s <= t) & ((t - s) % D == 0)
    loc = (s <= t) & (t - s < W)
    return np.concatenate([dil, loc], axis=1)


def attn_masked(q, ks, vs, kr, vr, D, W, scale):
    q = np.asarray(q, np.float64)
    B, T, H, d = q.shape
    if kr is None:
        kr = np.zeros_like(q)
        vr = np.zeros_like(q)
    out = np.zeros_like(q)
    D = np.broadcast_to(np.asarray(D), (H,))
    W = np.broadcast_to(np.asarray(W), (H,))
    for h in range(H):
        mask = attention_mask(T, int(D[h]), int(W[h]))
        for b in range(B):
            keys = np.concatenate([ks[b, :, h], kr[b, :, h]], axis=0)  # [2T, d]
            vals = np.concatenate([vs[b, :, h], vr[b, :, h]], axis=0)
            z = scale * (q[b, :, h] @ keys.T)  # [T, 2T]
            z = np.where(mask, z, -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, :, h] = p @ vals
    return out


def chunk_mask(T, D):
    """Boolean [T, T] mask of the chunk grid: key s is a chunk end
    (s mod D == D - 1) strictly before t, or t itself."""
    t = np.arange(T)[:, None]
    s = np.arange(T)[None, :]
    return ((s % D == D - 1) & (s < t)) | (s == t)


def chunk_attn_masked(q, ks, vs, D, scale):
    """Chunk-grid attention as one dense masked softmax per (b, h)."""
    q = np.asarray(q, np.float64)
    B, T, H, d = q.shape
    out = np.zeros_like(q)
    D = np.broadcast_to(np.asarray(D), (H,))
    for h in range(H):
        mask = chunk_mask(T, int(D[h]))
        for b in range(B):
            z = scale * (q[b, :, h] @ ks[b, :, h].T)
            z = np.where(mask, z, -np.inf)
            z = z - z.max(axis=1, keepdims=True)
            p = np.exp(z)
            p = p / p.sum(axis=1, keepdims=True)
            out[b, :, h] = p @ vs[b, :, h]
    return out
