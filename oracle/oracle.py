"""ctypes front end of the plain C oracle (``oracle.c``).

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, by the smoke check and by the
benchmark's CPU-baseline leg, never by the GPU library or its Python binding.

Every function takes and returns numpy float64 arrays (inputs are converted
with an exact widening cast, so bf16 / fp32 values are carried unchanged) and
follows the definitions documented at the top of ``oracle.c``:
"RAT+ Deep Dive" (zhichai.net) S1, S2.1, S3.1, S6 and the RAT+ abstract
(arXiv 2602.18196).

``Oracle(path)`` binds any compiled copy of ``oracle.c`` (the mutation tests
build deliberately broken copies to show that the pins catch them); the
module-level functions use the library built next to this file.
"""
from __future__ import annotations

import ctypes
import os
import subprocess

import numpy as np

_HERE = os.path.dirname(os.path.abspath(__file__))
SOURCE = os.path.join(_HERE, "oracle.c")
LIBRARY = os.path.join(_HERE, "liboracle.so")

MODE_RESTART = 0
MODE_SLIDING = 1


def compile_oracle(src: str, out: str) -> str:
    """Compile one C file into a shared library with the host compiler."""
    tmp = out + ".tmp"
    cmd = ["gcc", "-O2", "-std=c11", "-fopenmp", "-fPIC", "-shared",
           "-Wall", "-Werror", src, "-o", tmp, "-lm"]
    subprocess.run(cmd, check=True)
    os.replace(tmp, out)
    return out


def build(force: bool = True) -> str:
    """Compile oracle.c (no HIP headers, no GPU code)."""
    if force or not os.path.exists(LIBRARY):
        compile_oracle(SOURCE, LIBRARY)
    return LIBRARY


def _f64(a):
    if a is None:
        return None
    if hasattr(a, "detach"):  # torch tensor: widen on the CPU
        a = a.detach().to("cpu").double().numpy()
    return np.ascontiguousarray(np.asarray(a, dtype=np.float64))


def _ptr(a):
    if a is None:
        return None
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_double))


def _iptr(a):
    return a.ctypes.data_as(ctypes.POINTER(ctypes.c_int))


def _check(rc, name):
    if rc != 0:
        raise ValueError(f"{name} rejected its arguments (code {rc})")


def _heads(D, W, H):
    D = np.ascontiguousarray(np.broadcast_to(np.asarray(D, dtype=np.int32), (H,)))
    W = np.ascontiguousarray(np.broadcast_to(np.asarray(W, dtype=np.int32), (H,)))
    return D, W


class Oracle:
    """One loaded copy of the oracle library."""

    def __init__(self, path: str):
        lib = ctypes.CDLL(path)
        dp = ctypes.POINTER(ctypes.c_double)
        ip = ctypes.POINTER(ctypes.c_int)
        lp = ctypes.POINTER(ctypes.c_longlong)
        i, d = ctypes.c_int, ctypes.c_double
        lib.oracle_gates.argtypes = [dp, dp, dp, ctypes.c_long]
        lib.oracle_scan.argtypes = [dp, dp, dp, dp, dp, i, i, i, i, i, i]
        lib.oracle_index_sets.argtypes = [i, i, i, ip, ip, ip, ip]
        lib.oracle_index_sets.restype = ctypes.c_long
        lib.oracle_attn_prefill.argtypes = [dp, dp, dp, dp, dp, dp, i, i, i, i, ip, ip, d]
        lib.oracle_attn_prefill_rows.argtypes = [dp, dp, dp, dp, dp, ip, i, dp,
                                                 i, i, i, i, ip, ip, d]
        lib.oracle_attn_decode.argtypes = [dp, dp, dp, i, dp, dp, i, dp, i, i, i, i, ip, ip, d]
        lib.oracle_count_pairs.argtypes = [i, i, i, lp, lp]
        lib.oracle_chunk_index_set.argtypes = [i, i, ip]
        lib.oracle_chunk_index_set.restype = ctypes.c_long
        lib.oracle_chunk_attn_prefill_rows.argtypes = [dp, dp, dp, ip, i, dp, i, i, i, i, ip, d]
        lib.oracle_layer_backward.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                              i, i, i, i, i, i, ip, ip, d]
        lib.oracle_layer_backward_states.argtypes = [dp, dp, dp, dp, dp, dp, dp, dp, dp, dp, dp,
                                                     i, i, i, i, i, i, ip, ip, d]
        lib.oracle_num_threads.restype = ctypes.c_int
        self.lib = lib
        self.path = path

    def gates(self, logit):
        """(g, 1-g) = (sigmoid(l), sigmoid(-l)) elementwise."""
        x = _f64(logit)
        g = np.empty_like(x)
        gb = np.empty_like(x)
        _check(self.lib.oracle_gates(_ptr(x), _ptr(g), _ptr(gb), x.size), "oracle_gates")
        return g, gb

    def scan(self, k, v, logit, L, mode=MODE_RESTART):
        """Recurrent states (k_state, v_state) of [B,T,H,d] inputs."""
        k, v, logit = _f64(k), _f64(v), _f64(logit)
        B, T, H, d = k.shape
        ks = np.empty_like(k)
        vs = np.empty_like(v)
        _check(self.lib.oracle_scan(_ptr(k), _ptr(v), _ptr(logit), _ptr(ks), _ptr(vs),
                                    B, T, H, d, int(L), int(mode)), "oracle_scan")
        return ks, vs

    def index_sets(self, t, D, W):
        """(dilated positions, local positions) of query t, in oracle order."""
        nd, nl = ctypes.c_int(), ctypes.c_int()
        self.lib.oracle_index_sets(t, D, W, None, ctypes.byref(nd), None, ctypes.byref(nl))
        dil = np.empty(max(nd.value, 1), dtype=np.int32)
        loc = np.empty(max(nl.value, 1), dtype=np.int32)
        self.lib.oracle_index_sets(t, D, W, _iptr(dil), ctypes.byref(nd), _iptr(loc),
                                   ctypes.byref(nl))
        return dil[: nd.value].copy(), loc[: nl.value].copy()

    def num_threads(self):
        """OpenMP threads the oracle's parallel loops use."""
        return int(self.lib.oracle_num_threads())

    def count_pairs(self, T, D, W):
        """(sum_t |S_dil(t)|, sum_t |S_loc(t)|) over the T queries of one head."""
        a, b = ctypes.c_longlong(), ctypes.c_longlong()
        _check(self.lib.oracle_count_pairs(T, D, W, ctypes.byref(a), ctypes.byref(b)),
               "oracle_count_pairs")
        return a.value, b.value

    def attn_prefill(self, q, k_state, v_state, k_raw, v_raw, D, W, scale):
        """Prefill attention output [B,T,H,d] (every row)."""
        q, ks, vs = _f64(q), _f64(k_state), _f64(v_state)
        kr, vr = _f64(k_raw), _f64(v_raw)
        B, T, H, d = q.shape
        Da, Wa = _heads(D, W, H)
        out = np.empty_like(q)
        _check(self.lib.oracle_attn_prefill(_ptr(q), _ptr(ks), _ptr(vs), _ptr(kr), _ptr(vr),
                                            _ptr(out), B, T, H, d, _iptr(Da), _iptr(Wa),
                                            float(scale)), "oracle_attn_prefill")
        return out

    def attn_prefill_rows(self, q, k_state, v_state, k_raw, v_raw, rows, D, W, scale):
        """Prefill attention output for sampled rows [(b, t, h), ...] -> [n, d]."""
        q, ks, vs = _f64(q), _f64(k_state), _f64(v_state)
        kr, vr = _f64(k_raw), _f64(v_raw)
        B, T, H, d = q.shape
        Da, Wa = _heads(D, W, H)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        out = np.empty((r.shape[0], d), dtype=np.float64)
        _check(self.lib.oracle_attn_prefill_rows(_ptr(q), _ptr(ks), _ptr(vs), _ptr(kr),
                                                 _ptr(vr), _iptr(r), r.shape[0], _ptr(out),
                                                 B, T, H, d, _iptr(Da), _iptr(Wa),
                                                 float(scale)), "oracle_attn_prefill_rows")
        return out

    def chunk_index_set(self, t, D):
        """Chunk-grid keys of query t: chunk-end positions before t, then t."""
        n = int(self.lib.oracle_chunk_index_set(int(t), int(D), None))
        if n < 0:
            raise ValueError("oracle_chunk_index_set rejected its arguments")
        pos = np.empty(n, dtype=np.int32)
        self.lib.oracle_chunk_index_set(int(t), int(D), _iptr(pos))
        return pos

    def chunk_attn_prefill_rows(self, q, k_state, v_state, rows, D, scale):
        """Chunk-grid prefill attention for sampled rows [(b, t, h), ...] -> [n, d]."""
        q, ks, vs = _f64(q), _f64(k_state), _f64(v_state)
        B, T, H, d = q.shape
        Da, _ = _heads(D, 0, H)
        r = np.ascontiguousarray(np.asarray(rows, dtype=np.int32).reshape(-1, 3))
        out = np.empty((r.shape[0], d), dtype=np.float64)
        _check(self.lib.oracle_chunk_attn_prefill_rows(_ptr(q), _ptr(ks), _ptr(vs), _iptr(r),
                                                       r.shape[0], _ptr(out), B, T, H, d,
                                                       _iptr(Da), float(scale)),
               "oracle_chunk_attn_prefill_rows")
        return out

    def chunk_attn_prefill(self, q, k_state, v_state, D, scale):
        """Chunk-grid prefill attention, every row -> [B,T,H,d]."""
        B, T, H, d = q.shape
        rows = np.array([(b, t, h) for b in range(B) for t in range(T) for h in range(H)], np.int32)
        return self.chunk_attn_prefill_rows(q, k_state, v_state, rows, D, scale).reshape(B, T, H, d)

    def attn_decode(self, q, kd, vd, kw, vw, T, D, W, scale):
        """Decode output [B,H,d] at context length T."""
        q, kd, vd = _f64(q), _f64(kd), _f64(vd)
        kw, vw = _f64(kw), _f64(vw)
        B, H, d = q.shape
        nd_cap = kd.shape[2]
        w_cap = kw.shape[2] if kw is not None else 0
        Da, Wa = _heads(D, W, H)
        out = np.empty_like(q)
        _check(self.lib.oracle_attn_decode(_ptr(q), _ptr(kd), _ptr(vd), nd_cap, _ptr(kw),
                                           _ptr(vw), w_cap, _ptr(out), B, int(T), H, d,
                                           _iptr(Da), _iptr(Wa), float(scale)),
               "oracle_attn_decode")
        return out

    def layer_backward(self, q, k, v, logit, dout, L, mode, D, W, scale):
        """Gradients (dq, dk, dv, dlogit), each [B,T,H,d], of <dout, out>
        through the recurrence (full, RESTART or SLIDING) and the attention."""
        q, k, v, logit, dout = (_f64(x) for x in (q, k, v, logit, dout))
        B, T, H, d = q.shape
        Da, Wa = _heads(D, W, H)
        dq, dk, dv, dl = (np.empty_like(q) for _ in range(4))
        _check(self.lib.oracle_layer_backward(_ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(dout),
                                              _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dl), B, T, H, d,
                                              int(L), int(mode), _iptr(Da), _iptr(Wa), float(scale)),
               "oracle_layer_backward")
        return dq, dk, dv, dl

    def layer_backward_states(self, q, k, v, logit, k_state, v_state, dout, L, mode, D, W, scale):
        """The same gradients evaluated at given states (k_state, v_state),
        as a backward handed the forward's saved states computes them."""
        q, k, v, logit, ks, vs, dout = (_f64(x) for x in (q, k, v, logit, k_state, v_state, dout))
        B, T, H, d = q.shape
        Da, Wa = _heads(D, W, H)
        dq, dk, dv, dl = (np.empty_like(q) for _ in range(4))
        _check(self.lib.oracle_layer_backward_states(_ptr(q), _ptr(k), _ptr(v), _ptr(logit), _ptr(ks), _ptr(vs),
                                                     _ptr(dout), _ptr(dq), _ptr(dk), _ptr(dv), _ptr(dl), B, T, H,
                                                     d, int(L), int(mode), _iptr(Da), _iptr(Wa), float(scale)),
               "oracle_layer_backward_states")
        return dq, dk, dv, dl


_default = None


def default() -> Oracle:
    """The oracle built from ``oracle.c`` next to this file (built if missing)."""
    global _default
    if _default is None:
        if not os.path.exists(LIBRARY):
            build(force=False)
        _default = Oracle(LIBRARY)
    return _default


def gates(logit):
    return default().gates(logit)


def scan(k, v, logit, L, mode=MODE_RESTART):
    return default().scan(k, v, logit, L, mode)


def index_sets(t, D, W):
    return default().index_sets(t, D, W)


def count_pairs(T, D, W):
    return default().count_pairs(T, D, W)


def attn_prefill(q, k_state, v_state, k_raw, v_raw, D, W, scale):
    return default().attn_prefill(q, k_state, v_state, k_raw, v_raw, D, W, scale)


def attn_prefill_rows(q, k_state, v_state, k_raw, v_raw, rows, D, W, scale):
    return default().attn_prefill_rows(q, k_state, v_state, k_raw, v_raw, rows, D, W, scale)


def attn_decode(q, kd, vd, kw, vw, T, D, W, scale):
    return default().attn_decode(q, kd, vd, kw, vw, T, D, W, scale)


def chunk_index_set(t, D):
    return default().chunk_index_set(t, D)


def chunk_attn_prefill_rows(q, k_state, v_state, rows, D, scale):
    return default().chunk_attn_prefill_rows(q, k_state, v_state, rows, D, scale)


def chunk_attn_prefill(q, k_state, v_state, D, scale):
    return default().chunk_attn_prefill(q, k_state, v_state, D, scale)


def layer_backward(q, k, v, logit, dout, L, mode, D, W, scale):
    return default().layer_backward(q, k, v, logit, dout, L, mode, D, W, scale)


def layer_backward_states(q, k, v, logit, k_state, v_state, dout, L, mode, D, W, scale):
    return default().layer_backward_states(q, k, v, logit, k_state, v_state, dout, L, mode, D, W, scale)
