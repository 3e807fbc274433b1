"""GPU parity of chunk-grid prefill attention (the absolute reading of the
dilated pattern: each query sees the states ending a chunk of D tokens
before it, and its own state) against the fp64 oracle."""
import math

import numpy as np
import pytest
import torch

import dilated_sparse_attention_amd as rat
from oracle import oracle
from tests.parity import announce, assert_parity, guarded_empty, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _inputs(B, T, H, d, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    mk = lambda: torch.randn((B, T, H, d), generator=g).to(dtype)  # noqa: E731
    return mk(), mk(), mk()


CASES = [
    # (B, T, H, d, D per head, dtype)
    (1, 64, 1, 128, [1], torch.bfloat16),                # dense causal, one tile
    (1, 600, 2, 128, [1, 4], torch.bfloat16),            # several 256-row levels (pipelined tiles)
    (2, 300, 3, 64, [3, 16, 7], torch.bfloat16),         # ragged residues, d = 64
    (1, 1000, 2, 128, [1000, 1200], torch.bfloat16),     # D >= T: the own state only
    (1, 130, 2, 128, [64, 65], torch.bfloat16),          # one or two chunk ends
    (1, 2048, 2, 128, [16, 64], torch.bfloat16),
    (1, 256, 2, 64, [4, 4], torch.float32),
    (1, 200, 3, 128, [1, 5, 64], torch.float32),
]


@pytest.mark.parametrize("case", CASES, ids=lambda c: f"B{c[0]}T{c[1]}H{c[2]}d{c[3]}D{c[4]}{str(c[5])[6:]}")
def test_chunk_parity(case):
    B, T, H, d, D, dtype = case
    q, ks, vs = _inputs(B, T, H, d, dtype, 0)
    out, check = guarded_empty(q.shape, dtype)
    announce("chunk attn", (B, T, H, d), "D", D, dtype)
    rat.chunk_attn_prefill(q.cuda(), ks.cuda(), vs.cuda(), D=D, out=out)
    torch.cuda.synchronize()
    check()
    want = oracle.chunk_attn_prefill(q, ks, vs, D, 1 / math.sqrt(d))
    assert_parity(out, want, dtype, "chunk attn out")


def test_chunk_full_size_sampled():
    """The 1.5B layer shape (B=4, T=4096, H=16, d=128, D=16) on the chunk
    grid, in the launch configuration of the benchmark: sampled rows."""
    B, T, H, d, D = 4, 4096, 16, 128, 16
    q, ks, vs = _inputs(B, T, H, d, torch.bfloat16, 1)
    announce("chunk attn full size")
    out = rat.chunk_attn_prefill(q.cuda(), ks.cuda(), vs.cuda(), D=D)
    torch.cuda.synchronize()
    r = np.random.default_rng(2)
    rows = [(int(r.integers(B)), int(t), int(r.integers(H)))
            for t in list(r.integers(0, T, 200)) + [0, 14, 15, 16, 31, T - 1]]
    want = oracle.chunk_attn_prefill_rows(q, ks, vs, rows, D, 1 / math.sqrt(d))
    got = torch.stack([out[b, t, h] for (b, t, h) in rows])
    assert_parity(got, want, torch.bfloat16, "chunk attn sampled rows")


def test_chunk_last_residue_matches_relative():
    """Queries ending a chunk (t mod D = D - 1) see the same keys under both
    readings: the two GPU paths agree there."""
    q, ks, vs = (t.cuda() for t in _inputs(1, 1024, 2, 128, torch.bfloat16, 3))
    announce("chunk vs relative")
    a = rat.chunk_attn_prefill(q, ks, vs, D=[16, 4])
    b = rat.dilated_attn_prefill(q, ks, vs, D=[16, 4], W=[0, 0])
    for h, D in enumerate((16, 4)):
        x = a[0, D - 1::D, h].float()
        y = b[0, D - 1::D, h].float()
        assert (x - y).abs().max().item() <= 2e-2


def test_chunk_decode_cache():
    """A decode cache under the chunk grid -- the chunk ends before T-1 and
    the own state, ceil(T/D) rows -- read by the decode kernel unchanged,
    equals prefill row T-1."""
    B, T, H, d, D = 2, 777, 2, 128, [16, 64]
    q, ks, vs = _inputs(B, T, H, d, torch.bfloat16, 4)
    announce("chunk decode cache")
    pre = rat.chunk_attn_prefill(q.cuda(), ks.cuda(), vs.cuda(), D=D)
    n_cap = max((T - 1) // Dh + 1 for Dh in D)
    kd = torch.zeros((B, H, n_cap, d), dtype=torch.bfloat16)
    vd = torch.zeros_like(kd)
    for h, Dh in enumerate(D):
        pos = oracle.chunk_index_set(T - 1, Dh)
        kd[:, h, : len(pos)] = ks[:, pos, h]
        vd[:, h, : len(pos)] = vs[:, pos, h]
    out = rat.dilated_attn_decode(q[:, T - 1].contiguous().cuda(), kd.cuda(), vd.cuda(), None, None, T, D, [0, 0])
    torch.cuda.synchronize()
    want = oracle.chunk_attn_prefill_rows(q, ks, vs, [(b, T - 1, h) for b in range(B) for h in range(H)], D,
                                          1 / math.sqrt(d)).reshape(B, H, d)
    assert_parity(out, want, torch.bfloat16, "chunk decode")
    assert (out.float() - pre[:, T - 1].float()).abs().max().item() <= 2e-2
