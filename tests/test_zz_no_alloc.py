"""The decode entry point that allocates nothing
(rat_dilated_attn_decode_static): through the C ABI, its output equals
rat_dilated_attn_decode's with a caller workspace, bit for bit, on two
calls in a row -- the second smaller than the first, so it runs over what
the first left in the shared static scratch -- and on a call that needs no
split partials at all."""
import pytest
import torch

import dilated_sparse_attention_amd as rat
from tests.parity import announce, requires_gpu

pytestmark = [pytest.mark.gpu, requires_gpu]


def _case(B, H, d, T, D, W, dtype, seed):
    g = torch.Generator().manual_seed(seed)
    nd_cap = max((T - 1) // Dh + 1 for Dh in D)
    w_cap = max(max(W), 1)
    mk = lambda *s: torch.randn(s, generator=g).to(dtype).cuda()  # noqa: E731
    return (mk(B, H, d), mk(B, H, nd_cap, d), mk(B, H, nd_cap, d), mk(B, H, w_cap, d), mk(B, H, w_cap, d))


CASES = [
    # (B, H, d, T, D per head, W per head, dtype): the first two split their
    # keys over many workgroups (partials in the scratch), the last does not
    (1, 4, 128, 20000, [1, 4, 16, 64], [0, 64, 0, 128], torch.bfloat16),
    (2, 2, 64, 3000, [2, 8], [16, 0], torch.float32),
    (64, 20, 128, 32768, [64] * 20, [64] * 20, torch.bfloat16),
]


def test_static_decode_matches_workspace_decode():
    lib = rat.load_library()
    assert lib.rat_decode_static_scratch_bytes() == 1 << 20
    for i, (B, H, d, T, D, W, dtype) in enumerate(CASES):
        announce("static decode", i, (B, H, d, T), "D", D, "W", W, dtype)
        q, kd, vd, kw, vw = _case(B, H, d, T, D, W, dtype, seed=40 + i)
        need = rat.decode_workspace_bytes(B, H, d, T, D, W)
        assert (need > 0) == (i < 2), need
        assert need <= lib.rat_decode_static_scratch_bytes()
        want = rat.dilated_attn_decode(q, kd, vd, kw, vw, T, D, W)
        got = rat.dilated_attn_decode_static(q, kd, vd, kw, vw, T, D, W)
        again = rat.dilated_attn_decode_static(q, kd, vd, kw, vw, T, D, W)
        torch.cuda.synchronize()
        assert torch.isfinite(want.float()).all()
        assert torch.equal(got, want), f"case {i}: max diff {(got.float() - want.float()).abs().max():.3g}"
        assert torch.equal(again, want)
