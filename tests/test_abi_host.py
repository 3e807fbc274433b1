"""The C-ABI library on the host (no GPU): it loads, exports every symbol
``include/rat.h`` declares, sizes workspaces, and rejects invalid arguments
with the documented status codes before touching the HIP runtime."""
import ctypes
import os
import re

import pytest

from dilated_sparse_attention_amd import ops

ROOT = os.path.dirname(os.path.dirname(os.path.abspath(__file__)))
HEADER = os.path.join(ROOT, "include", "rat.h")

OK, NULL, SHAPE, UNSUP, ALIAS, WSPACE, HIP, ALIGN = range(8)


@pytest.fixture(scope="module")
def lib():
    if not os.path.exists(ops.LIBRARY):
        from dilated_sparse_attention_amd import build
        build.build()
    return ops.load_library()


def declared_functions():
    text = open(HEADER).read()
    text = re.sub(r"/\*.*?\*/", "", text, flags=re.S)
    return sorted(set(re.findall(r"\b(rat_[a-z_0-9]+)\s*\(", text)))


def test_header_and_binding_agree():
    assert declared_functions() == sorted(ops.EXPORTS)


def test_every_declared_symbol_is_exported(lib):
    for name in declared_functions():
        assert hasattr(lib, name), name


def test_status_strings(lib):
    for code in range(8):
        assert lib.rat_status_string(code)
    assert lib.rat_status_string(99) == b"unknown status"
    assert lib.rat_last_hip_error() == 0


# fake, 256-byte aligned "device" addresses: validation must reject every
# case below before any of them is dereferenced or handed to HIP
P = [ctypes.c_void_p(0x10000 + 0x100000 * i) for i in range(8)]
MIS = ctypes.c_void_p(0x10008)


def heads(vals):
    return (ctypes.c_int * len(vals))(*vals)


def scan(lib, k=P[0], v=P[1], g=P[2], ks=P[3], vs=P[4], B=1, T=64, H=2, d=64, L=64, mode=0, dtype=1,
         ws=P[5], wsb=1 << 30, fin=None):
    return lib.rat_scan_prefill(k, v, g, ks, vs, B, T, H, d, L, mode, dtype, ws, wsb, fin, None)


def test_scan_final_state_validation(lib):
    assert scan(lib, T=200, L=64, mode=1, fin=P[6]) == UNSUP  # SLIDING keeps no single state
    assert scan(lib, fin=P[3]) == ALIAS
    assert scan(lib, fin=MIS) == ALIGN


def test_scan_validation(lib):
    assert scan(lib, k=None) == NULL
    assert scan(lib, vs=None) == NULL
    assert scan(lib, B=0) == SHAPE
    assert scan(lib, T=-1) == SHAPE
    assert scan(lib, L=0) == SHAPE
    assert scan(lib, mode=7) == SHAPE
    assert scan(lib, d=96) == UNSUP
    assert scan(lib, dtype=5) == UNSUP
    assert scan(lib, B=1 << 10, T=1 << 12, H=64, d=128) == UNSUP  # >= 2^31 elements
    assert scan(lib, T=1000, L=100, mode=1) == UNSUP  # SLIDING window above 64
    assert scan(lib, ks=P[0]) == ALIAS
    assert scan(lib, vs=P[3]) == ALIAS
    assert scan(lib, k=MIS) == ALIGN
    assert scan(lib, ws=None) == WSPACE
    assert scan(lib, wsb=16) == WSPACE
    assert scan(lib, ws=ctypes.c_void_p(0x10040)) == WSPACE  # not 256-byte aligned


def test_scan_workspace_sizes(lib):
    # full and RESTART need a workspace; a SLIDING window needs none
    assert lib.rat_scan_workspace_bytes(4, 4096, 16, 128, 4096, 0, 1) > 0
    assert lib.rat_scan_workspace_bytes(1, 16384, 16, 128, 64, 0, 1) > 0
    assert lib.rat_scan_workspace_bytes(1, 16384, 16, 128, 64, 1, 1) == 0
    assert lib.rat_scan_workspace_bytes(1, 100, 2, 64, 1000, 1, 1) > 0  # L >= T: full
    assert lib.rat_scan_workspace_bytes(0, 100, 2, 64, 100, 0, 1) == 0
    small = lib.rat_scan_workspace_bytes(1, 256, 2, 64, 256, 0, 1)
    big = lib.rat_scan_workspace_bytes(2, 4096, 2, 64, 4096, 0, 1)
    assert 256 <= small < big


def attn(lib, q=P[0], ks=P[1], vs=P[2], kr=P[3], vr=P[4], out=P[5], B=1, T=64, H=2, d=128,
         D=(4, 4), W=(0, 8), scale=0.1, dtype=1, ws=P[6], wsb=1 << 30):
    Dh = None if D is None else heads(D)
    Wh = None if W is None else heads(W)
    return lib.rat_dilated_attn_prefill(q, ks, vs, kr, vr, out, B, T, H, d, Dh, Wh, scale, dtype, ws, wsb, None)


def test_attn_validation(lib):
    assert attn(lib, q=None) == NULL
    assert attn(lib, out=None) == NULL
    assert attn(lib, kr=None) == NULL  # head 1 has a window
    assert attn(lib, D=None) == NULL
    assert attn(lib, T=0) == SHAPE
    assert attn(lib, D=(0, 4)) == SHAPE
    assert attn(lib, W=(0, -1)) == SHAPE
    assert attn(lib, d=32) == UNSUP
    assert attn(lib, dtype=3) == UNSUP
    assert attn(lib, scale=float("nan")) == SHAPE
    assert attn(lib, out=P[1]) == ALIAS
    assert attn(lib, out=P[3]) == ALIAS
    assert attn(lib, vs=MIS) == ALIGN
    H = 300
    assert attn(lib, H=H, D=[1] * H, W=[0] * H) == UNSUP  # more heads than the kernel table
    many = [(i % 9) + 1 for i in range(16)]
    assert attn(lib, H=16, D=many, W=[0] * 16) == UNSUP  # more than 8 (D, W) classes
    # a head with a window needs the partial-state workspace
    assert attn(lib, ws=None) == WSPACE
    assert attn(lib, wsb=8) == WSPACE


def test_attn_workspace_sizes(lib):
    assert lib.rat_attn_prefill_workspace_bytes(1, 64, 2, 128, heads([4, 4]), heads([0, 8]), 1) == 64 * 2 * 8
    assert lib.rat_attn_prefill_workspace_bytes(4, 4096, 16, 128, heads([16] * 16), heads([0] * 16), 1) == 0
    assert lib.rat_attn_prefill_workspace_bytes(1, 64, 2, 128, heads([4, 4]), heads([0, 8]), 0) == 0  # fp32


def chunk(lib, q=P[0], ks=P[1], vs=P[2], out=P[5], B=1, T=64, H=2, d=128, D=(4, 16), scale=0.1, dtype=1):
    Dh = None if D is None else heads(D)
    return lib.rat_chunk_attn_prefill(q, ks, vs, out, B, T, H, d, Dh, scale, dtype, None)


def test_chunk_attn_validation(lib):
    assert chunk(lib, q=None) == NULL
    assert chunk(lib, vs=None) == NULL
    assert chunk(lib, D=None) == NULL
    assert chunk(lib, T=0) == SHAPE
    assert chunk(lib, D=(0, 4)) == SHAPE
    assert chunk(lib, d=32) == UNSUP
    assert chunk(lib, dtype=3) == UNSUP
    assert chunk(lib, scale=float("nan")) == SHAPE
    assert chunk(lib, out=P[1]) == ALIAS
    assert chunk(lib, ks=MIS) == ALIGN
    assert chunk(lib, H=300, D=[4] * 300) == UNSUP
    many = [(i % 9) + 1 for i in range(16)]
    assert chunk(lib, H=16, D=many) == UNSUP  # more than 8 dilation classes


def decode(lib, q=P[0], kd=P[1], vd=P[2], nd_cap=512, kw=P[3], vw=P[4], w_cap=64, out=P[5], B=4, T=32768,
           H=2, d=128, D=(64, 64), W=(64, 64), scale=0.1, dtype=1, ws=P[6], wsb=1 << 30):
    return lib.rat_dilated_attn_decode(q, kd, vd, nd_cap, kw, vw, w_cap, out, B, T, H, d, heads(D), heads(W),
                                       scale, dtype, ws, wsb, None)


def test_decode_validation(lib):
    assert decode(lib, q=None) == NULL
    assert decode(lib, kw=None) == NULL
    assert decode(lib, T=0) == SHAPE
    assert decode(lib, nd_cap=511) == SHAPE  # ceil(32768 / 64) = 512 entries needed
    assert decode(lib, w_cap=63) == SHAPE
    assert decode(lib, D=(64, 0)) == SHAPE
    assert decode(lib, d=256) == UNSUP
    assert decode(lib, out=P[2]) == ALIAS
    assert decode(lib, kd=MIS) == ALIGN
    # one long head, few pairs: split-key partials need a workspace
    need = lib.rat_decode_workspace_bytes(1, 1, 128, 1 << 20, heads([1]), heads([0]))
    assert need > 0
    assert decode(lib, B=1, H=1, T=1 << 20, D=(1,), W=(0,), nd_cap=1 << 20, w_cap=0, ws=None) == WSPACE
    assert lib.rat_decode_workspace_bytes(64, 20, 128, 32768, heads([64] * 20), heads([64] * 20)) == 0
    # a cache of more than 2^31 elements passes the size checks (64-bit
    # cache offsets): the misaligned query is the first error found
    assert decode(lib, q=MIS, B=64, H=20, D=[64] * 20, W=[64] * 20, nd_cap=1 << 15) == ALIGN
    assert decode(lib, nd_cap=1 << 24) == UNSUP  # one head's rows exceed 2^31 elements


def step(lib, q=P[0], kn=P[1], vn=P[2], gn=P[3], st=P[4], kc=P[5], vc=P[6], n_cap=1024, kw=P[7],
         vw=ctypes.c_void_p(0x10000 + 0x100000 * 9), w_cap=64, out=ctypes.c_void_p(0x10000 + 0x100000 * 10),
         B=2, T=1000, H=2, d=128, L=1 << 30, D=(64, 16), W=(64, 0), scale=0.1, dtype=1,
         ws=ctypes.c_void_p(0x10000 + 0x100000 * 11), wsb=1 << 30):
    return lib.rat_decode_step(q, kn, vn, gn, st, kc, vc, n_cap, kw, vw, w_cap, out, B, T, H, d, L, heads(D),
                               heads(W), scale, dtype, ws, wsb, None)


def test_decode_step_validation(lib):
    assert step(lib, st=None) == NULL
    assert step(lib, kw=None) == NULL          # head 0 has a window
    assert step(lib, L=0) == SHAPE
    assert step(lib, w_cap=63) == SHAPE        # ring slot (T-1) mod 64 needs 64 slots
    # position 999 of the D = 64 head sits at row 15 of its residue: 16 rows per residue needed
    assert step(lib, n_cap=64 * 15) == SHAPE
    assert step(lib, d=32) == UNSUP
    assert step(lib, out=P[0]) == ALIAS
    assert step(lib, kc=P[1]) == ALIAS
    assert step(lib, vc=P[5]) == ALIAS
    assert step(lib, st=MIS) == ALIGN
    # the full-position history of a 64 x 20-head batch at T = 32768 (> 2^31 elements)
    assert step(lib, st=MIS, B=64, H=20, n_cap=1 << 15, T=32768, D=[64] * 20, W=[64] * 20) == ALIGN


def layer(lib, q=P[0], k=P[1], v=P[2], g=P[3], out=P[4], kc=P[5], vc=P[6], n_cap=1024, kw=P[7],
          vw=ctypes.c_void_p(0x10000 + 0x100000 * 9), w_cap=64, fin=None, B=1, T=1000, H=2, d=128, L=1000,
          mode=0, D=(64, 16), W=(64, 0), scale=0.1, dtype=1, sws=ctypes.c_void_p(0x10000 + 0x100000 * 10),
          swsb=1 << 30, aws=ctypes.c_void_p(0x10000 + 0x100000 * 11), awsb=1 << 30):
    return lib.rat_layer_prefill(q, k, v, g, out, kc, vc, n_cap, kw, vw, w_cap, fin, B, T, H, d, L, mode,
                                 heads(D), heads(W), scale, dtype, sws, swsb, aws, awsb, None)


def test_layer_prefill_validation(lib):
    assert layer(lib, kc=None) == NULL
    assert layer(lib, kw=None) == NULL                 # head 0 has a window
    assert layer(lib, n_cap=0) == SHAPE
    # position 999 of the D = 64 head is row 15 of its residue: 16 rows per residue needed
    assert layer(lib, n_cap=64 * 15) == SHAPE
    assert layer(lib, w_cap=63) == SHAPE               # ring slots p mod 64
    assert layer(lib, mode=5) == SHAPE
    assert layer(lib, d=32) == UNSUP
    assert layer(lib, B=64, H=20, D=[64] * 20, W=[64] * 20, n_cap=1 << 15) == UNSUP  # history >= 2^31 elements
    assert layer(lib, mode=1, L=64, fin=ctypes.c_void_p(0x10000 + 0x100000 * 12)) == UNSUP  # SLIDING: no state
    assert layer(lib, mode=1, L=100) == UNSUP          # SLIDING window above 64
    assert layer(lib, out=P[0]) == ALIAS
    assert layer(lib, kc=P[1]) == ALIAS
    assert layer(lib, vw=P[5]) == ALIAS                # two outputs share memory
    assert layer(lib, fin=P[6]) == ALIAS
    assert layer(lib, vc=MIS) == ALIGN
    assert layer(lib, sws=None) == WSPACE              # the full recurrence needs its workspace
    assert layer(lib, sws=ctypes.c_void_p(0x10040)) == WSPACE
    assert layer(lib, aws=None) == WSPACE              # a windowed head needs the attention workspace


def backward(lib, q=P[0], k=P[1], v=P[2], g=P[3], ks=P[4], vs=P[5], dout=P[7],
             dq=ctypes.c_void_p(0x10000 + 0x100000 * 9), dk=ctypes.c_void_p(0x10000 + 0x100000 * 10),
             dv=ctypes.c_void_p(0x10000 + 0x100000 * 11), dg=ctypes.c_void_p(0x10000 + 0x100000 * 12),
             B=1, T=100, H=2, d=128, L=100, mode=0, D=(1, 64), W=(0, 8), scale=0.1, dtype=1,
             ws=ctypes.c_void_p(0x10000 + 0x100000 * 13), wsb=1 << 30):
    return lib.rat_layer_backward(q, k, v, g, ks, vs, dout, dq, dk, dv, dg, B, T, H, d, L, mode,
                                  heads(D), heads(W), scale, dtype, ws, wsb, None)


def test_backward_validation(lib):
    assert backward(lib, dout=None) == NULL
    assert backward(lib, dg=None) == NULL
    assert backward(lib, T=0) == SHAPE
    assert backward(lib, D=(0, 1)) == SHAPE
    assert backward(lib, d=96) == UNSUP
    assert backward(lib, mode=1, L=64, dq=P[0]) == ALIAS  # a SLIDING window validates like the rest
    assert backward(lib, mode=2) == SHAPE            # no such recurrence mode
    assert backward(lib, dq=P[0]) == ALIAS
    assert backward(lib, dv=ctypes.c_void_p(0x10000 + 0x100000 * 9)) == ALIAS  # two gradients share memory
    assert backward(lib, ks=MIS) == ALIGN
    assert backward(lib, ws=None) == WSPACE
    assert backward(lib, wsb=1024) == WSPACE


def test_backward_workspace_size(lib):
    B, T, H, d = 2, 100, 3, 64
    rows, elems = B * T * H, B * T * H * d
    cells = ((T + 15) // 16) * B * H * d
    need = lib.rat_layer_backward_workspace_bytes(B, T, H, d)
    # per row lse, delta and the raw window's three partial sums; the state
    # gradients; per chunk cell the maps (5) and carries (4); seven parts
    # each 256-byte aligned
    assert need >= 4 * (5 * rows + 2 * elems + 9 * cells)
    assert need < 4 * (5 * rows + 2 * elems + 9 * cells) + 7 * 256
    assert lib.rat_layer_backward_workspace_bytes(0, T, H, d) == 0


def caches(lib, ks=P[0], vs=P[1], k=P[2], v=P[3], kc=P[4], vc=P[5], n_cap=1024, kw=P[6], vw=P[7], w_cap=64,
           B=1, T=1000, H=2, d=128, D=(64, 16), W=(64, 0), dtype=1):
    return lib.rat_build_decode_caches(ks, vs, k, v, kc, vc, n_cap, kw, vw, w_cap, B, T, H, d, heads(D), heads(W),
                                       dtype, None)


def test_build_decode_caches_validation(lib):
    assert caches(lib, kc=None) == NULL
    assert caches(lib, kw=None) == NULL           # head 0 has a window
    assert caches(lib, n_cap=64 * 15) == SHAPE    # position 999 of D = 64 needs 16 rows per residue
    assert caches(lib, w_cap=63) == SHAPE
    assert caches(lib, d=48) == UNSUP
    assert caches(lib, kc=P[0]) == ALIAS
    assert caches(lib, vw=P[6]) == ALIAS
    assert caches(lib, vc=MIS) == ALIGN


def test_cached_workspaces_are_per_stream(monkeypatch):
    """The binding's cached scan / attention workspaces are keyed by
    (device, stream): calls in flight on two streams never share one."""
    import torch

    class Stream:
        def __init__(self, handle):
            self.cuda_stream = handle

    current = {"s": Stream(11)}
    monkeypatch.setattr(ops.torch.cuda, "current_stream", lambda device=None: current["s"])
    monkeypatch.setattr(ops.torch.cuda, "current_device", lambda: 0)
    real_zeros, real_empty = torch.zeros, torch.empty
    monkeypatch.setattr(ops.torch, "zeros", lambda *a, **k: real_zeros(*a, **dict(k, device="cpu")))
    monkeypatch.setattr(ops.torch, "empty", lambda *a, **k: real_empty(*a, **dict(k, device="cpu")))
    monkeypatch.setattr(ops, "_workspaces", {})
    monkeypatch.setattr(ops, "_attn_workspaces", {})
    for get in (ops.scan_workspace, ops.attn_workspace):
        current["s"] = Stream(11)
        a = get(4096, "cuda:0")
        assert get(1024, "cuda:0") is a                 # same stream: reused
        current["s"] = Stream(12)
        b = get(4096, "cuda:0")
        assert b is not a and b.data_ptr() != a.data_ptr()  # another stream: its own buffer
        current["s"] = Stream(11)
        assert get(4096, "cuda:0") is a
        assert get(1 << 16, "cuda:0").numel() >= 1 << 16  # grown on demand


def test_static_decode_validation(lib):
    """The decode entry point without a workspace validates like the one
    with: errors before any HIP call (the fake pointers are never touched)."""
    assert lib.rat_decode_static_scratch_bytes() == 1 << 20
    D, W = heads([4, 4]), heads([0, 8])

    def call(q=P[0], kd=P[1], vd=P[2], nd=64, kw=P[3], vw=P[4], wc=8, out=P[5], B=1, T=100, H=2, d=64, Dh=D, Wh=W,
             scale=0.125, dtype=1):
        return lib.rat_dilated_attn_decode_static(q, kd, vd, nd, kw, vw, wc, out, B, T, H, d, Dh, Wh, scale, dtype,
                                                  None)

    assert call(q=None) == NULL
    assert call(kw=None) == NULL
    assert call(B=0) == SHAPE
    assert call(nd=10) == SHAPE      # ceil(100 / 4) = 25 entries needed
    assert call(wc=4) == SHAPE       # min(W, T) = 8 ring slots needed
    assert call(d=96) == UNSUP
    assert call(dtype=5) == UNSUP
    assert call(out=P[0]) == ALIAS
    assert call(q=MIS) == ALIGN
    assert call(scale=float("nan")) == SHAPE


def test_sliding_decode_validation(lib):
    """The SLIDING decode step and its state fill validate before any HIP call."""
    D, W = heads([4, 4]), heads([0, 8])

    X = [ctypes.c_void_p(0x2000000 + 0x100000 * i) for i in range(4)]  # q, k_new, v_new, gate_new

    def step(q=X[0], rk=P[1], rv=P[2], rg=P[3], L=64, kc=P[4], vc=P[5], n_cap=128, kw=P[6], vw=P[7], w_cap=8,
             out=P[0], B=1, T=100, H=2, d=64, scale=0.125, dtype=1):
        return lib.rat_decode_step_sliding(q, X[1], X[2], X[3], rk, rv, rg, L, kc, vc, n_cap, kw, vw, w_cap, out,
                                           B, T, H, d, D, W, scale, dtype, None, 0, None)

    assert step(q=None) == NULL
    assert step(rg=None) == NULL
    assert step(kw=None) == NULL
    assert step(L=0) == SHAPE
    assert step(L=1025) == UNSUP
    assert step(n_cap=16) == SHAPE      # (T-1) / 4 = 24 needs n_cap / 4 > 24
    assert step(w_cap=4) == SHAPE
    assert step(d=96) == UNSUP
    assert step(rk=P[2]) == ALIAS        # two outputs share memory
    assert step(out=X[0]) == ALIAS       # an output is the query
    assert step(rk=MIS) == ALIGN
    assert step(scale=float("nan")) == SHAPE

    def fill(k=P[0], v=P[1], g=P[2], rk=P[3], rv=P[4], rg=P[5], B=1, T=100, H=2, d=64, L=64, dtype=1):
        return lib.rat_sliding_state_from_prefill(k, v, g, rk, rv, rg, B, T, H, d, L, dtype, None)

    assert fill(g=None) == NULL
    assert fill(T=0) == SHAPE
    assert fill(L=0) == SHAPE
    assert fill(L=2000) == UNSUP
    assert fill(d=32) == UNSUP
    assert fill(rk=P[0]) == ALIAS
    assert fill(rg=P[3]) == ALIAS
    assert fill(rv=MIS) == ALIGN
