"""Seeded synthetic inputs for the CARVE chunk forward pass.

This module only draws random numbers and casts them to a storage dtype. It
holds none of the layer's arithmetic, so the GPU path and the CPU oracle can
both consume its output without sharing any method code.

Distributions (the same for every workload):
  q, k      N(0,1), then L2-normalised per (batch, token, head) row
  v         N(0,1)
  g         -softplus(N(0,1)) per key dimension (a log-decay, always <= 0)
  bx        N(0,1) per key dimension (erase logit)
  w         sigmoid(N(0,1)) per (batch, token, head) (scalar write gate)
  U_down    N(0, ub_std) of shape [H, rank, dv]
  U_up      N(0, ub_std) of shape [H, dk, rank]
Draw order is fixed: q, k, v, g, bx, w, U_down, U_up, all from one
numpy PCG64 generator in float64, then each tensor is cast once to the storage
dtype with round-to-nearest-even (bf16 goes through float32 first).

Activation-layer tensors use the token-major layout [B, T, H, d] that a
fused q/k/v/gate projection produces; w is [B, T, H].
"""
from __future__ import annotations

from dataclasses import dataclass, replace

import numpy as np

__all__ = [
    "Workload", "WORKLOADS", "make_inputs", "bf16_bits_from_f32",
    "f64_from_bf16_bits", "to_f64",
]


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    T: int
    dk: int
    dv: int
    L: int
    dtype: str          # "f32" or "bf16": storage and operand type
    rank: int           # rank of the content projection U_b; 0 = absent
    ub_std: float
    seed: int

    @property
    def head_tokens(self) -> int:
        return self.B * self.T * self.H

    def tag(self) -> str:
        """File-name tag, e.g. B4H12T2048_d64_L64_bf16 (plus _r16 with a content projection)."""
        return f"B{self.B}H{self.H}T{self.T}_d{self.dk}_L{self.L}_{self.dtype}" + (f"_r{self.rank}" if self.rank else "")

    def describe(self) -> str:
        return (f"B={self.B} H={self.H} T={self.T} d_k={self.dk} d_v={self.dv} L={self.L} {self.dtype}, "
                + (f"content projection rank {self.rank}" if self.rank else "no content projection"))

    def with_(self, **kw) -> "Workload":
        return replace(self, **kw)


WORKLOADS = {
    # tiny fp32 case with a live content path
    "tiny": Workload("tiny", 1, 2, 256, 64, 64, 64, "f32", 8, 0.02, 1001),
    # headline shape: content projection absent
    "init_equiv": Workload("init_equiv", 4, 12, 2048, 64, 64, 64, "bf16", 0, 0.0, 1002),
    "content": Workload("content", 8, 12, 4096, 64, 64, 64, "bf16", 16, 0.05, 1003),
    # chunk-size sweep: the same inputs are run at L in {16, 32, 64, 128}
    "lsweep": Workload("lsweep", 4, 16, 8192, 128, 128, 64, "bf16", 16, 0.05, 1004),
    "long": Workload("long", 1, 16, 65536, 128, 128, 64, "bf16", 16, 0.05, 1005),
    # fp32 case whose content projection is large enough to move the output
    # far beyond the fp32 tolerance, so parity proves the content path runs
    "content_test": Workload("content_test", 1, 2, 1024, 64, 64, 64, "f32", 16, 1.0, 1006),
    # decode steps: one token of 64 x 12 (batch, head) pairs per step; T is the
    # number of distinct tokens drawn (one chunk), cycled by the benchmark
    "decode": Workload("decode", 64, 12, 64, 64, 64, 64, "bf16", 16, 0.05, 1007),
}
LSWEEP_CHUNKS = (16, 32, 64, 128)


def bf16_bits_from_f32(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); return uint16 bit patterns."""
    u = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    rounded = (u + 0x7FFF + ((u >> 16) & 1)) >> 16
    out = rounded.astype(np.uint16)
    nan = np.isnan(x)
    if nan.any():
        out[nan] = 0x7FC0
    return out


def f64_from_bf16_bits(bits: np.ndarray) -> np.ndarray:
    return (bits.astype(np.uint32) << 16).view(np.float32).astype(np.float64)


def _cast(x64: np.ndarray, dtype: str) -> np.ndarray:
    x32 = x64.astype(np.float32)
    if dtype == "f32":
        return x32
    if dtype == "bf16":
        return bf16_bits_from_f32(x32)
    raise ValueError(f"unknown dtype {dtype!r}")


def to_f64(stored: np.ndarray, dtype: str) -> np.ndarray:
    """Exact float64 upcast of a tensor produced by make_inputs."""
    if dtype == "f32":
        return stored.astype(np.float64)
    return f64_from_bf16_bits(stored)


def _softplus(x: np.ndarray) -> np.ndarray:
    return np.maximum(x, 0.0) + np.log1p(np.exp(-np.abs(x)))


def _sigmoid(x: np.ndarray) -> np.ndarray:
    return 0.5 * (1.0 + np.tanh(0.5 * x))


def make_inputs(wl: Workload, decay_logits: bool = False) -> dict:
    """Draw one workload's inputs. Returns storage arrays (float32, or uint16 bf16 bits).

    Keys: q, k, v, g, bx, w, and U_down, U_up when wl.rank > 0. With
    decay_logits, g holds the raw N(0,1) draws themselves (the decay logits,
    before the activation) instead of -softplus of them; every other tensor
    and the draw order are unchanged.
    """
    rng = np.random.Generator(np.random.PCG64(wl.seed))
    B, T, H, dk, dv = wl.B, wl.T, wl.H, wl.dk, wl.dv
    out = {}

    def draw(shape):
        return rng.standard_normal(shape)

    for name in ("q", "k"):
        x = draw((B, T, H, dk))
        x /= np.sqrt(np.sum(x * x, axis=-1, keepdims=True))
        out[name] = _cast(x, wl.dtype)
        del x
    out["v"] = _cast(draw((B, T, H, dv)), wl.dtype)
    a = draw((B, T, H, dk))
    out["g"] = _cast(a if decay_logits else -_softplus(a), wl.dtype)
    del a
    out["bx"] = _cast(draw((B, T, H, dk)), wl.dtype)
    out["w"] = _cast(_sigmoid(draw((B, T, H))), wl.dtype)
    if wl.rank > 0:
        out["U_down"] = _cast(wl.ub_std * draw((H, wl.rank, dv)), wl.dtype)
        out["U_up"] = _cast(wl.ub_std * draw((H, dk, wl.rank)), wl.dtype)
    return out


def to_torch(stored: np.ndarray, dtype: str, device="cuda"):
    """Move a storage array from make_inputs to a torch tensor (bf16 bits become torch.bfloat16)."""
    import torch
    if dtype == "f32":
        return torch.from_numpy(np.ascontiguousarray(stored)).to(device)
    t = torch.from_numpy(np.ascontiguousarray(stored).view(np.int16))
    return t.view(torch.bfloat16).to(device)
