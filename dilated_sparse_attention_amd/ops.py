"""Python binding of the RAT+ C ABI (``include/rat.h``) on torch tensors.

Argument marshalling only: every step runs in the HIP library ``librat.so``
that sits next to this file.  There is no CPU fallback; if the library is
missing or no GPU is present the calls raise.  Tensors must be contiguous
CUDA (ROCm) tensors; work is enqueued on torch's current stream.
"""
from __future__ import annotations

import ctypes
import math
import os

import torch

_HERE = os.path.dirname(os.path.abspath(__file__))
LIBRARY = os.path.join(_HERE, "librat.so")

RESTART = 0
SLIDING = 1

_DTYPES = {torch.float32: 0, torch.bfloat16: 1}

STATUS = {0: "RAT_OK", 1: "RAT_ERR_NULL", 2: "RAT_ERR_SHAPE", 3: "RAT_ERR_UNSUPPORTED",
          4: "RAT_ERR_ALIAS", 5: "RAT_ERR_WORKSPACE", 6: "RAT_ERR_HIP", 7: "RAT_ERR_ALIGN"}

# every symbol include/rat.h declares
EXPORTS = ("rat_scan_workspace_bytes", "rat_scan_prefill", "rat_attn_prefill_workspace_bytes", "rat_dilated_attn_prefill",
           "rat_chunk_attn_prefill",
           "rat_decode_workspace_bytes", "rat_decode_step", "rat_dilated_attn_decode", "rat_layer_prefill",
           "rat_decode_static_scratch_bytes", "rat_dilated_attn_decode_static",
           "rat_decode_step_sliding", "rat_sliding_state_from_prefill",
           "rat_layer_backward_workspace_bytes", "rat_layer_backward", "rat_build_decode_caches",
           "rat_status_string",
           "rat_last_hip_error")


class RatError(RuntimeError):
    def __init__(self, fn, code, lib):
        msg = lib.rat_status_string(code).decode()
        extra = ""
        if code == 6:
            extra = f" (hipError {lib.rat_last_hip_error()})"
        super().__init__(f"{fn} failed: {STATUS.get(code, code)}: {msg}{extra}")
        self.code = code


_lib = None


def load_library(path: str = LIBRARY):
    """Load librat.so and declare the C signatures (raises if absent)."""
    global _lib
    if _lib is not None and path == LIBRARY:
        return _lib
    if not os.path.exists(path):
        raise RuntimeError(f"{path} is missing: build it with `python -m dilated_sparse_attention_amd.build`; "
                           "there is no CPU fallback")
    lib = ctypes.CDLL(path)
    vp, i, sz, f = ctypes.c_void_p, ctypes.c_int, ctypes.c_size_t, ctypes.c_float
    ip = ctypes.POINTER(ctypes.c_int)
    lib.rat_scan_workspace_bytes.argtypes = [i, i, i, i, i, i, i]
    lib.rat_scan_workspace_bytes.restype = sz
    lib.rat_scan_prefill.argtypes = [vp, vp, vp, vp, vp, i, i, i, i, i, i, i, vp, sz, vp, vp]
    lib.rat_scan_prefill.restype = i
    lib.rat_attn_prefill_workspace_bytes.argtypes = [i, i, i, i, ip, ip, i]
    lib.rat_attn_prefill_workspace_bytes.restype = sz
    lib.rat_dilated_attn_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, ip, ip, f, i, vp, sz, vp]
    lib.rat_dilated_attn_prefill.restype = i
    lib.rat_chunk_attn_prefill.argtypes = [vp, vp, vp, vp, i, i, i, i, ip, f, i, vp]
    lib.rat_chunk_attn_prefill.restype = i
    lib.rat_decode_workspace_bytes.argtypes = [i, i, i, i, ip, ip]
    lib.rat_decode_workspace_bytes.restype = sz
    lib.rat_dilated_attn_decode.argtypes = [vp, vp, vp, i, vp, vp, i, vp, i, i, i, i, ip, ip, f, i, vp, sz, vp]
    lib.rat_dilated_attn_decode.restype = i
    lib.rat_decode_static_scratch_bytes.argtypes = []
    lib.rat_decode_static_scratch_bytes.restype = sz
    lib.rat_dilated_attn_decode_static.argtypes = [vp, vp, vp, i, vp, vp, i, vp, i, i, i, i, ip, ip, f, i, vp]
    lib.rat_dilated_attn_decode_static.restype = i
    lib.rat_decode_step_sliding.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, i, vp, vp, i, vp, i, i, i, i, ip,
                                            ip, f, i, vp, sz, vp]
    lib.rat_decode_step_sliding.restype = i
    lib.rat_sliding_state_from_prefill.argtypes = [vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, vp]
    lib.rat_sliding_state_from_prefill.restype = i
    lib.rat_decode_step.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, i, vp, i, i, i, i, i, ip, ip, f, i, vp, sz,
                                    vp]
    lib.rat_decode_step.restype = i
    lib.rat_layer_prefill.argtypes = [vp, vp, vp, vp, vp, vp, vp, i, vp, vp, i, vp, i, i, i, i, i, i, ip, ip, f, i,
                                      vp, sz, vp, sz, vp]
    lib.rat_layer_prefill.restype = i
    lib.rat_build_decode_caches.argtypes = [vp, vp, vp, vp, vp, vp, i, vp, vp, i, i, i, i, i, ip, ip, i, vp]
    lib.rat_build_decode_caches.restype = i
    lib.rat_layer_backward_workspace_bytes.argtypes = [i, i, i, i]
    lib.rat_layer_backward_workspace_bytes.restype = sz
    lib.rat_layer_backward.argtypes = [vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, vp, i, i, i, i, i, i, ip, ip, f, i,
                                       vp, sz, vp]
    lib.rat_layer_backward.restype = i
    lib.rat_status_string.argtypes = [i]
    lib.rat_status_string.restype = ctypes.c_char_p
    lib.rat_last_hip_error.argtypes = []
    lib.rat_last_hip_error.restype = i
    if path == LIBRARY:
        _lib = lib
    return lib


def _ptr(t):
    return None if t is None else ctypes.c_void_p(t.data_ptr())


def _stream():
    return ctypes.c_void_p(torch.cuda.current_stream().cuda_stream)


def _heads(x, H):
    vals = list(x) if hasattr(x, "__len__") else [int(x)] * H
    if len(vals) != H:
        raise ValueError(f"expected {H} per-head values, got {len(vals)}")
    return (ctypes.c_int * H)(*[int(v) for v in vals])


def _check_tensor(name, t, dtype, shape=None):
    if t is None:
        return
    if not t.is_cuda:
        raise ValueError(f"{name} must be a GPU tensor")
    if t.dtype != dtype:
        raise ValueError(f"{name} has dtype {t.dtype}, expected {dtype}")
    if not t.is_contiguous():
        raise ValueError(f"{name} must be contiguous")
    if shape is not None and tuple(t.shape) != tuple(shape):
        raise ValueError(f"{name} has shape {tuple(t.shape)}, expected {tuple(shape)}")


def _raise(fn, rc, lib):
    if rc != 0:
        raise RatError(fn, rc, lib)


# ------------------------------------------------------------------ scan
def scan_workspace_bytes(B, T, H, d, L, mode=RESTART, dtype=torch.bfloat16):
    return int(load_library().rat_scan_workspace_bytes(B, T, H, d, L, mode, _DTYPES[dtype]))


_workspaces = {}


def _ws_key(device):
    """Cached workspaces are kept per (device, stream): calls in flight on
    two streams must not share one (the scan's carries and tickets assume
    one call at a time per workspace)."""
    dev = torch.device(device)
    idx = dev.index if dev.index is not None else torch.cuda.current_device()
    return idx, torch.cuda.current_stream(idx).cuda_stream


def scan_workspace(nbytes, device):
    """A zero-filled scan workspace of at least ``nbytes`` on ``device``,
    kept per (device, current stream) and reused (the library keeps it
    consistent itself)."""
    key = _ws_key(device)
    ws = _workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.zeros(max(nbytes, 256), dtype=torch.uint8, device=device)
        _workspaces[key] = ws
    return ws


def scan_prefill(k, v, gate_logits, L=None, mode=RESTART, k_state=None, v_state=None, workspace=None,
                 final_state=None):
    """Recurrent states (k_state, v_state) of [B,T,H,d] keys / values with
    forget-gate logits ``gate_logits`` (L defaults to T: full recurrence).
    ``final_state`` (fp32 [B,H,2,d]) receives the states at T-1 unrounded."""
    lib = load_library()
    B, T, H, d = k.shape
    L = T if L is None else int(L)
    for name, t in (("k", k), ("v", v), ("gate_logits", gate_logits)):
        _check_tensor(name, t, k.dtype, k.shape)
    k_state = torch.empty_like(k) if k_state is None else k_state
    v_state = torch.empty_like(v) if v_state is None else v_state
    _check_tensor("k_state", k_state, k.dtype, k.shape)
    _check_tensor("v_state", v_state, k.dtype, k.shape)
    nbytes = lib.rat_scan_workspace_bytes(B, T, H, d, L, mode, _DTYPES[k.dtype])
    if workspace is None and nbytes:
        workspace = scan_workspace(nbytes, k.device)
    if final_state is not None:
        _check_tensor("final_state", final_state, torch.float32, (B, H, 2, d))
    rc = lib.rat_scan_prefill(_ptr(k), _ptr(v), _ptr(gate_logits), _ptr(k_state), _ptr(v_state),
                              B, T, H, d, L, mode, _DTYPES[k.dtype], _ptr(workspace),
                              0 if workspace is None else workspace.numel(), _ptr(final_state), _stream())
    _raise("rat_scan_prefill", rc, lib)
    return k_state, v_state


# ------------------------------------------------------------------ attention
def attn_prefill_workspace_bytes(B, T, H, d, D, W, dtype=torch.bfloat16):
    return int(load_library().rat_attn_prefill_workspace_bytes(B, T, H, d, _heads(D, H), _heads(W, H),
                                                               _DTYPES[dtype]))


_attn_workspaces = {}


def attn_workspace(nbytes, device):
    """Scratch for the local-window pass of prefill attention (no
    initialisation needed), kept per (device, current stream) and grown on
    demand."""
    key = _ws_key(device)
    ws = _attn_workspaces.get(key)
    if ws is None or ws.numel() < nbytes:
        ws = torch.empty(max(nbytes, 256), dtype=torch.uint8, device=device)
        _attn_workspaces[key] = ws
    return ws


def dilated_attn_prefill(q, k_state, v_state, k_raw=None, v_raw=None, D=1, W=0, scale=None, out=None,
                         workspace=None):
    """Dilated (+ local window) causal attention over the recurrent states."""
    lib = load_library()
    B, T, H, d = q.shape
    for name, t in (("q", q), ("k_state", k_state), ("v_state", v_state), ("k_raw", k_raw), ("v_raw", v_raw)):
        _check_tensor(name, t, q.dtype, q.shape)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.dtype, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    Dh, Wh = _heads(D, H), _heads(W, H)
    nbytes = lib.rat_attn_prefill_workspace_bytes(B, T, H, d, Dh, Wh, _DTYPES[q.dtype])
    if workspace is None and nbytes:
        workspace = attn_workspace(nbytes, q.device)
    rc = lib.rat_dilated_attn_prefill(_ptr(q), _ptr(k_state), _ptr(v_state), _ptr(k_raw), _ptr(v_raw),
                                      _ptr(out), B, T, H, d, Dh, Wh, scale, _DTYPES[q.dtype], _ptr(workspace),
                                      0 if workspace is None else workspace.numel(), _stream())
    _raise("rat_dilated_attn_prefill", rc, lib)
    return out


def chunk_attn_prefill(q, k_state, v_state, D=1, scale=None, out=None):
    """Chunk-grid causal attention: each query sees the states that end a
    chunk of D tokens before it, and its own state."""
    lib = load_library()
    B, T, H, d = q.shape
    for name, t in (("q", q), ("k_state", k_state), ("v_state", v_state)):
        _check_tensor(name, t, q.dtype, q.shape)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.dtype, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    rc = lib.rat_chunk_attn_prefill(_ptr(q), _ptr(k_state), _ptr(v_state), _ptr(out), B, T, H, d, _heads(D, H),
                                    scale, _DTYPES[q.dtype], _stream())
    _raise("rat_chunk_attn_prefill", rc, lib)
    return out


def decode_workspace_bytes(B, H, d, T, D, W):
    return int(load_library().rat_decode_workspace_bytes(B, H, d, T, _heads(D, H), _heads(W, H)))


def dilated_attn_decode(q, kd, vd, kw, vw, T, D, W, scale=None, out=None, workspace=None):
    """Decode attention of the query at position T-1 over the dilated cache
    (kd, vd: [B,H,nd_cap,d]) and the raw ring (kw, vw: [B,H,w_cap,d])."""
    lib = load_library()
    B, H, d = q.shape
    _check_tensor("q", q, q.dtype)
    _check_tensor("kd", kd, q.dtype)
    _check_tensor("vd", vd, q.dtype, kd.shape)
    _check_tensor("kw", kw, q.dtype)
    _check_tensor("vw", vw, q.dtype, None if kw is None else kw.shape)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.dtype, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    Dh, Wh = _heads(D, H), _heads(W, H)
    nbytes = lib.rat_decode_workspace_bytes(B, H, d, int(T), Dh, Wh)
    if workspace is None and nbytes:
        workspace = torch.empty(nbytes, dtype=torch.uint8, device=q.device)
    w_cap = 0 if kw is None else kw.shape[2]
    rc = lib.rat_dilated_attn_decode(_ptr(q), _ptr(kd), _ptr(vd), kd.shape[2], _ptr(kw), _ptr(vw), w_cap,
                                     _ptr(out), B, int(T), H, d, Dh, Wh, scale, _DTYPES[q.dtype],
                                     _ptr(workspace), 0 if workspace is None else workspace.numel(),
                                     _stream())
    _raise("rat_dilated_attn_decode", rc, lib)
    return out


def dilated_attn_decode_static(q, kd, vd, kw, vw, T, D, W, scale=None, out=None):
    """dilated_attn_decode without a workspace: the library keeps the split
    partials in its own static per-GPU scratch (calls overlapping on one GPU
    race; see rat_dilated_attn_decode_static)."""
    lib = load_library()
    B, H, d = q.shape
    _check_tensor("q", q, q.dtype)
    _check_tensor("kd", kd, q.dtype)
    _check_tensor("vd", vd, q.dtype, kd.shape)
    _check_tensor("kw", kw, q.dtype)
    _check_tensor("vw", vw, q.dtype, None if kw is None else kw.shape)
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.dtype, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    w_cap = 0 if kw is None else kw.shape[2]
    rc = lib.rat_dilated_attn_decode_static(_ptr(q), _ptr(kd), _ptr(vd), kd.shape[2], _ptr(kw), _ptr(vw), w_cap,
                                            _ptr(out), B, int(T), H, d, _heads(D, H), _heads(W, H), scale,
                                            _DTYPES[q.dtype], _stream())
    _raise("rat_dilated_attn_decode_static", rc, lib)
    return out


def prefill_two_calls(q, k, v, gate_logits, D, W, L=None, mode=RESTART, scale=None):
    """The whole prefill hot path as two library calls: rat_scan_prefill,
    then rat_dilated_attn_prefill over its states (the one-call C entry
    point that also emits decode caches is ``layer_prefill``)."""
    ks, vs = scan_prefill(k, v, gate_logits, L=L, mode=mode)
    need_raw = any(int(w) > 0 for w in (W if hasattr(W, "__len__") else [W]))
    return dilated_attn_prefill(q, ks, vs, k if need_raw else None, v if need_raw else None,
                                D=D, W=W, scale=scale)


def history_rows(T, D):
    """Rows per head a state history needs to hold positions 0 .. T-1 for
    every head's dilation: the smallest n with (T-1) // D[h] < n // D[h]."""
    return max(Dh * ((T - 1) // Dh + 1) for Dh in D)


def layer_prefill(q, k, v, gate_logits, D, W, L=None, mode=RESTART, scale=None, n_cap=None, w_cap=None,
                  final_state=True, out=None, kc=None, vc=None, kw=None, vw=None):
    """The whole prefill (recurrence, then dilated + local attention) in one
    library call, emitting the decode caches: the per-residue state history
    (kc, vc: [B,H,n_cap,d]), the raw ring of the last W tokens (kw, vw:
    [B,H,w_cap,d]) and the fp32 states at T-1.  ``n_cap`` defaults to the
    rows positions 0 .. T-1 need.  Returns (out, kc, vc, kw, vw, state);
    kw / vw are None when every W is 0, state None when not asked for."""
    lib = load_library()
    B, T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("gate_logits", gate_logits)):
        _check_tensor(name, t, q.dtype, q.shape)
    L = T if L is None else int(L)
    Dl = list(D) if hasattr(D, "__len__") else [int(D)] * H
    Wl = list(W) if hasattr(W, "__len__") else [int(W)] * H
    Dh, Wh = _heads(Dl, H), _heads(Wl, H)
    n_cap = history_rows(T, Dl) if n_cap is None else int(n_cap)
    if kc is None:
        kc = torch.empty((B, H, n_cap, d), dtype=q.dtype, device=q.device)
    if vc is None:
        vc = torch.empty_like(kc)
    _check_tensor("kc", kc, q.dtype, (B, H, n_cap, d))
    _check_tensor("vc", vc, q.dtype, (B, H, n_cap, d))
    any_w = any(int(x) > 0 for x in Wl)
    w_cap = (max(int(x) for x in Wl) if any_w else 0) if w_cap is None else int(w_cap)
    if any_w and kw is None:
        kw = torch.zeros((B, H, w_cap, d), dtype=q.dtype, device=q.device)
    if any_w and vw is None:
        vw = torch.zeros_like(kw)
    if kw is not None:
        _check_tensor("kw", kw, q.dtype, (B, H, w_cap, d))
        _check_tensor("vw", vw, q.dtype, (B, H, w_cap, d))
    if final_state is True:
        final_state = torch.empty((B, H, 2, d), dtype=torch.float32, device=q.device)
    elif final_state is False:
        final_state = None
    if final_state is not None:
        _check_tensor("final_state", final_state, torch.float32, (B, H, 2, d))
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.dtype, q.shape)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    sbytes = lib.rat_scan_workspace_bytes(B, T, H, d, L, mode, _DTYPES[q.dtype])
    sws = scan_workspace(sbytes, q.device) if sbytes else None
    abytes = lib.rat_attn_prefill_workspace_bytes(B, T, H, d, Dh, Wh, _DTYPES[q.dtype])
    aws = attn_workspace(abytes, q.device) if abytes else None
    rc = lib.rat_layer_prefill(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_logits), _ptr(out), _ptr(kc), _ptr(vc), n_cap,
                               _ptr(kw), _ptr(vw), w_cap, _ptr(final_state), B, T, H, d, L, mode, Dh, Wh, scale,
                               _DTYPES[q.dtype], _ptr(sws), 0 if sws is None else sws.numel(), _ptr(aws),
                               0 if aws is None else aws.numel(), _stream())
    _raise("rat_layer_prefill", rc, lib)
    return out, kc, vc, kw, vw, final_state


def build_decode_caches(k_state, v_state, k, v, D, W, n_cap=None, w_cap=None, kc=None, vc=None, kw=None, vw=None):
    """Decode caches of a finished prefill: the per-residue state history
    (kc, vc: [B,H,n_cap,d]) and the raw ring of the last W tokens (kw, vw:
    [B,H,w_cap,d]), as decode_step reads and extends them.  Returns
    (kc, vc, kw, vw); kw / vw are None when every W is 0."""
    lib = load_library()
    B, T, H, d = k_state.shape
    for name, t in (("k_state", k_state), ("v_state", v_state), ("k", k), ("v", v)):
        _check_tensor(name, t, k_state.dtype, k_state.shape)
    Dl = list(D) if hasattr(D, "__len__") else [int(D)] * H
    Wl = list(W) if hasattr(W, "__len__") else [int(W)] * H
    n_cap = history_rows(T, Dl) if n_cap is None else int(n_cap)
    kc = torch.empty((B, H, n_cap, d), dtype=k_state.dtype, device=k_state.device) if kc is None else kc
    vc = torch.empty_like(kc) if vc is None else vc
    _check_tensor("kc", kc, k_state.dtype, (B, H, n_cap, d))
    _check_tensor("vc", vc, k_state.dtype, (B, H, n_cap, d))
    any_w = any(int(x) > 0 for x in Wl)
    w_cap = (max(int(x) for x in Wl) if any_w else 0) if w_cap is None else int(w_cap)
    if any_w and kw is None:
        kw = torch.zeros((B, H, w_cap, d), dtype=k_state.dtype, device=k_state.device)
        vw = torch.zeros_like(kw)
    if kw is not None:
        _check_tensor("kw", kw, k_state.dtype, (B, H, w_cap, d))
        _check_tensor("vw", vw, k_state.dtype, (B, H, w_cap, d))
    rc = lib.rat_build_decode_caches(_ptr(k_state), _ptr(v_state), _ptr(k), _ptr(v), _ptr(kc), _ptr(vc), n_cap,
                                     _ptr(kw), _ptr(vw), w_cap, B, T, H, d, _heads(Dl, H), _heads(Wl, H),
                                     _DTYPES[k_state.dtype], _stream())
    _raise("rat_build_decode_caches", rc, lib)
    return kc, vc, kw, vw


def layer_backward(q, k, v, gate_logits, k_state, v_state, dout, D, W, L=None, mode=RESTART, scale=None,
                   grads=None, workspace=None):
    """Gradients (dq, dk, dv, dgate), fp32 [B,T,H,d], of a loss with
    incoming gradient ``dout`` through the layer's forward (the states it
    produced are passed in).  Full recurrence, RESTART or a SLIDING window."""
    lib = load_library()
    B, T, H, d = q.shape
    for name, t in (("q", q), ("k", k), ("v", v), ("gate_logits", gate_logits), ("k_state", k_state),
                    ("v_state", v_state), ("dout", dout)):
        _check_tensor(name, t, q.dtype, q.shape)
    if grads is None:
        grads = tuple(torch.empty(q.shape, dtype=torch.float32, device=q.device) for _ in range(4))
    for name, t in zip(("dq", "dk", "dv", "dgate"), grads):
        _check_tensor(name, t, torch.float32, q.shape)
    L = T if L is None else int(L)
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    nbytes = lib.rat_layer_backward_workspace_bytes(B, T, H, d)
    if workspace is None:
        workspace = attn_workspace(nbytes, q.device)
    rc = lib.rat_layer_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(gate_logits), _ptr(k_state), _ptr(v_state),
                                _ptr(dout), *(_ptr(g) for g in grads), B, T, H, d, L, mode,
                                _heads(D, H), _heads(W, H), scale, _DTYPES[q.dtype], _ptr(workspace),
                                workspace.numel(), _stream())
    _raise("rat_layer_backward", rc, lib)
    return grads


def decode_step(q, k_new, v_new, gate_new, state, kc, vc, kw, vw, T, D, W, L=None, scale=None, out=None,
                workspace=None):
    """One decode-loop step at context length T (the new token at position
    T-1): advances the fp32 ``state`` [B,H,2,d] by the token's (k_new, v_new,
    gate_new), writes its state into the per-residue history (kc, vc:
    [B,H,n_cap,d]) and its raw key / value into the ring (kw, vw:
    [B,H,w_cap,d]), then attends as dilated_attn_decode."""
    lib = load_library()
    B, H, d = q.shape
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("gate_new", gate_new)):
        _check_tensor(name, t, q.dtype, (B, H, d))
    _check_tensor("state", state, torch.float32, (B, H, 2, d))
    n_cap = kc.shape[2]
    _check_tensor("kc", kc, q.dtype, (B, H, n_cap, d))
    _check_tensor("vc", vc, q.dtype, (B, H, n_cap, d))
    w_cap = 0 if kw is None else kw.shape[2]
    if kw is not None:
        _check_tensor("kw", kw, q.dtype, (B, H, w_cap, d))
        _check_tensor("vw", vw, q.dtype, (B, H, w_cap, d))
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.dtype, (B, H, d))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    L = int(T) if L is None else int(L)
    Dh, Wh = _heads(D, H), _heads(W, H)
    nbytes = lib.rat_decode_workspace_bytes(B, H, d, int(T), Dh, Wh)
    if workspace is None and nbytes:
        workspace = attn_workspace(nbytes, q.device)
    rc = lib.rat_decode_step(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(gate_new), _ptr(state), _ptr(kc), _ptr(vc),
                             n_cap, _ptr(kw), _ptr(vw), w_cap, _ptr(out), B, int(T), H, d, L, Dh, Wh, scale,
                             _DTYPES[q.dtype], _ptr(workspace), 0 if workspace is None else workspace.numel(),
                             _stream())
    _raise("rat_decode_step", rc, lib)
    return out


def decode_step_sliding(q, k_new, v_new, gate_new, rk, rv, rg, kc, vc, kw, vw, T, D, W, scale=None, out=None,
                        workspace=None):
    """One decode-loop step at context length T under a SLIDING recurrence
    window of L = rk.shape[2] tokens: the new state is the recurrence from
    zero over the ring (rk, rv, rg: [B,H,L,d], raw key / value / gate logit
    of position p in slot p mod L) plus the new token, which takes its slot;
    then as decode_step (history kc, vc; raw ring kw, vw; attention)."""
    lib = load_library()
    B, H, d = q.shape
    for name, t in (("q", q), ("k_new", k_new), ("v_new", v_new), ("gate_new", gate_new)):
        _check_tensor(name, t, q.dtype, (B, H, d))
    L = rk.shape[2]
    for name, t in (("rk", rk), ("rv", rv), ("rg", rg)):
        _check_tensor(name, t, q.dtype, (B, H, L, d))
    n_cap = kc.shape[2]
    _check_tensor("kc", kc, q.dtype, (B, H, n_cap, d))
    _check_tensor("vc", vc, q.dtype, (B, H, n_cap, d))
    w_cap = 0 if kw is None else kw.shape[2]
    if kw is not None:
        _check_tensor("kw", kw, q.dtype, (B, H, w_cap, d))
        _check_tensor("vw", vw, q.dtype, (B, H, w_cap, d))
    out = torch.empty_like(q) if out is None else out
    _check_tensor("out", out, q.dtype, (B, H, d))
    scale = 1.0 / math.sqrt(d) if scale is None else float(scale)
    Dh, Wh = _heads(D, H), _heads(W, H)
    nbytes = lib.rat_decode_workspace_bytes(B, H, d, int(T), Dh, Wh)
    if workspace is None and nbytes:
        workspace = attn_workspace(nbytes, q.device)
    rc = lib.rat_decode_step_sliding(_ptr(q), _ptr(k_new), _ptr(v_new), _ptr(gate_new), _ptr(rk), _ptr(rv),
                                     _ptr(rg), L, _ptr(kc), _ptr(vc), n_cap, _ptr(kw), _ptr(vw), w_cap, _ptr(out),
                                     B, int(T), H, d, Dh, Wh, scale, _DTYPES[q.dtype], _ptr(workspace),
                                     0 if workspace is None else workspace.numel(), _stream())
    _raise("rat_decode_step_sliding", rc, lib)
    return out


def sliding_state_from_prefill(k, v, gate_logits, L, rk=None, rv=None, rg=None):
    """The SLIDING decode state of a finished prefill: the raw key, value and
    gate logit of its last L positions into rings [B,H,L,d] (slot p mod L).
    Returns (rk, rv, rg)."""
    lib = load_library()
    B, T, H, d = k.shape
    for name, t in (("k", k), ("v", v), ("gate_logits", gate_logits)):
        _check_tensor(name, t, k.dtype, k.shape)
    L = int(L)
    rk = torch.zeros((B, H, L, d), dtype=k.dtype, device=k.device) if rk is None else rk
    rv = torch.zeros_like(rk) if rv is None else rv
    rg = torch.zeros_like(rk) if rg is None else rg
    for name, t in (("rk", rk), ("rv", rv), ("rg", rg)):
        _check_tensor(name, t, k.dtype, (B, H, L, d))
    rc = lib.rat_sliding_state_from_prefill(_ptr(k), _ptr(v), _ptr(gate_logits), _ptr(rk), _ptr(rv), _ptr(rg),
                                            B, T, H, d, L, _DTYPES[k.dtype], _stream())
    _raise("rat_sliding_state_from_prefill", rc, lib)
    return rk, rv, rg
