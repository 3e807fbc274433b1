"""Seeded synthetic workloads: shapes, per-head (D, W), recurrence window and
value distributions of the RAT+ layer at the model scales the pages discuss.

This module only draws random numbers and lays them out; it holds none of the
layer's arithmetic.  Both the GPU tests and the CPU oracle tests take their
inputs from here.

Recipe (every workload): one ``torch.Generator('cpu')`` seeded with ``seed``;
fp32 ``torch.randn`` draws in the order listed by ``draw_order``; each draw is
shifted / scaled as the workload states; then cast to the workload dtype with
round-to-nearest-even (``Tensor.to``).  Gate tensors hold forget-gate LOGITS
(the layer applies the sigmoid itself).

Model scales follow the RAT+ abstract (arXiv 2602.18196: 1.5B, 2.6B and 7.6B
models) and "RAT+ Deep Dive" S3.1 (D = 16, 64), S2.3 / S6 (local windows of
16..1024 tokens), S6 Head-Wise Hybrid (dense heads beside dilated heads),
S7.3 (medium-long contexts of 4K-64K tokens).  The per-head shapes (H, d) are
typical of those model sizes; the pages do not print them.
"""
from __future__ import annotations

import math
from dataclasses import dataclass

import torch

MODE_RESTART = 0
MODE_SLIDING = 1


@dataclass(frozen=True)
class PrefillWorkload:
    name: str
    B: int
    T: int
    H: int
    d: int
    D: tuple  # per-head dilation
    W: tuple  # per-head local window (raw tokens)
    L: int  # recurrence window; L >= T means full-sequence recurrence
    dtype: torch.dtype
    qkv_std: float  # q, k, v ~ N(0, qkv_std^2)
    gate_mean: float  # gate logits ~ N(gate_mean, 1)
    modes: tuple = (MODE_RESTART,)
    draw_order: tuple = ("q", "k", "v", "gate")

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "T": self.T, "H": self.H, "d": self.d,
                "D": list(self.D), "W": list(self.W), "L": self.L,
                "dtype": str(self.dtype).replace("torch.", "")}


@dataclass(frozen=True)
class DecodeWorkload:
    name: str
    B: int
    T: int  # context length including the new token
    H: int
    d: int
    D: tuple
    W: tuple
    dtype: torch.dtype
    draw_order: tuple = ("q", "kd", "vd", "kw", "vw")

    @property
    def scale(self) -> float:
        return 1.0 / math.sqrt(self.d)

    @property
    def nd_cap(self) -> int:
        return max((self.T + Dh - 1) // Dh for Dh in self.D)

    @property
    def w_cap(self) -> int:
        return max(min(Wh, self.T) for Wh in self.W)

    def describe(self) -> dict:
        return {"workload": self.name, "B": self.B, "T": self.T, "H": self.H, "d": self.d,
                "D": list(self.D), "W": list(self.W), "dtype": str(self.dtype).replace("torch.", "")}


def _heads(value, H):
    return tuple([value] * H)


# Tiny fp32 prefill: parity case the oracle finishes instantly.
TINY_FP32 = PrefillWorkload(
    name="prefill_tiny_fp32_B1_T256_H2_d64_D4", B=1, T=256, H=2, d=64,
    D=_heads(4, 2), W=_heads(0, 2), L=256, dtype=torch.float32,
    qkv_std=1.0, gate_mean=2.0)

# 1.5B-scale layer (hidden 2048): the headline prefill workload.
PREFILL_1P5B = PrefillWorkload(
    name="prefill_1.5B_B4_T4096_H16_d128_D16", B=4, T=4096, H=16, d=128,
    D=_heads(16, 16), W=_heads(0, 16), L=4096, dtype=torch.bfloat16,
    qkv_std=1.0 / math.sqrt(128), gate_mean=2.0)

# Long prefill with a local window and the 64-token recurrence window.
PREFILL_LONG = PrefillWorkload(
    name="prefill_long_B1_T16384_H16_d128_D64_W128_L64", B=1, T=16384, H=16, d=128,
    D=_heads(64, 16), W=_heads(128, 16), L=64, dtype=torch.bfloat16,
    qkv_std=1.0, gate_mean=1.0, modes=(MODE_RESTART, MODE_SLIDING))

# 7.6B-scale head-wise hybrid (hidden 4096): 8 dense heads + 24 dilated heads.
PREFILL_7P6B_HYBRID = PrefillWorkload(
    name="prefill_7.6B_hybrid_B1_T32768_H32_d128_dense8_D64_W256", B=1, T=32768, H=32, d=128,
    D=tuple([1] * 8 + [64] * 24), W=tuple([0] * 8 + [256] * 24), L=32768,
    dtype=torch.bfloat16, qkv_std=1.0, gate_mean=2.0)

# 2.6B-scale batched decode (hidden 2560) at a 32768-token context.
DECODE_2P6B_D64 = DecodeWorkload(
    name="decode_2.6B_B64_T32768_H20_d128_D64_W64", B=64, T=32768, H=20, d=128,
    D=_heads(64, 20), W=_heads(64, 20), dtype=torch.bfloat16)

DECODE_2P6B_D16 = DecodeWorkload(
    name="decode_2.6B_B64_T32768_H20_d128_D16_W64", B=64, T=32768, H=20, d=128,
    D=_heads(16, 20), W=_heads(64, 20), dtype=torch.bfloat16)

PREFILL_WORKLOADS = (TINY_FP32, PREFILL_1P5B, PREFILL_LONG, PREFILL_7P6B_HYBRID)
DECODE_WORKLOADS = (DECODE_2P6B_D64, DECODE_2P6B_D16)


def _randn(gen, shape, device="cpu"):
    return torch.randn(shape, generator=gen, dtype=torch.float32, device=device)


def make_prefill(w: PrefillWorkload, seed: int = 0, device: str = "cpu", *, B=None, T=None):
    """q, k, v, gate logits as [B,T,H,d] tensors in ``w.dtype``.

    ``B`` / ``T`` override the workload's sizes (reduced parity cases keep
    every other property of the workload).  ``device='cuda'`` draws with a
    CUDA generator (same distribution, different stream) for benchmarking.
    """
    B = w.B if B is None else B
    T = w.T if T is None else T
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (B, T, w.H, w.d)
    out = {}
    for name in w.draw_order:
        x = _randn(gen, shape, device)
        if name == "gate":
            x = x + w.gate_mean
        else:
            x = x * w.qkv_std
        out[name] = x.to(w.dtype)
    return out


def make_decode(w: DecodeWorkload, seed: int = 0, device: str = "cpu", *, B=None):
    """q [B,H,d]; dilated caches kd, vd [B,H,nd_cap,d]; rings kw, vw [B,H,w_cap,d]."""
    B = w.B if B is None else B
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shapes = {"q": (B, w.H, w.d), "kd": (B, w.H, w.nd_cap, w.d), "vd": (B, w.H, w.nd_cap, w.d),
              "kw": (B, w.H, w.w_cap, w.d), "vw": (B, w.H, w.w_cap, w.d)}
    return {name: _randn(gen, shapes[name], device).to(w.dtype) for name in w.draw_order}


def make_random_prefill(B, T, H, d, dtype, seed, qkv_std=1.0, gate_mean=2.0, device="cpu"):
    """Free-form seeded prefill inputs for property sweeps."""
    gen = torch.Generator(device=device)
    gen.manual_seed(seed)
    shape = (B, T, H, d)
    q = (_randn(gen, shape, device) * qkv_std).to(dtype)
    k = (_randn(gen, shape, device) * qkv_std).to(dtype)
    v = (_randn(gen, shape, device) * qkv_std).to(dtype)
    g = (_randn(gen, shape, device) + gate_mean).to(dtype)
    return {"q": q, "k": k, "v": v, "gate": g}


def sha256_of(tensors: dict) -> dict:
    """SHA-256 of each tensor's bytes (contiguous, on the CPU), by name: the
    fingerprint of a drawn workload."""
    import hashlib

    out = {}
    for name, t in tensors.items():
        c = t.detach().contiguous().cpu()
        out[name] = hashlib.sha256(c.view(torch.uint8).numpy().tobytes()).hexdigest()
    return out
