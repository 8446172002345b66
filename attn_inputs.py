"""Seeded synthetic inputs for exact attention, as 16-bit bit patterns.

This module is shared by the CPU oracle's tests and by the GPU path's tests
and benchmark. It holds no attention arithmetic: it only draws i.i.d. normal
samples and rounds them to bfloat16, so that both sides see identical bits.

Recipe (the same for every workload):
  * generator: ``numpy.random.default_rng(seed)`` (PCG64);
  * each tensor: ``standard_normal(shape, float32) * sigma``, then
    round-to-nearest-even to bfloat16 (or, when asked, to IEEE binary16),
    kept as ``uint16`` bit patterns;
  * draw order: Q, K, V, then dO (only when gradients are wanted).

The five workloads are the shapes the "RTX Flash Attention Implementation
COMPLETE" page tabulates under "Performance Specifications" (Small, Medium,
Large, XL), with the modes and value distributions fixed for this library.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


@dataclass(frozen=True)
class Workload:
    name: str
    B: int
    H: int
    N: int
    d: int
    causal_modes: tuple      # which causal flags the workload runs
    backward: bool           # whether dO is drawn and gradients checked
    sigma_qk: float          # std of Q and K entries
    sigma_v: float           # std of V and dO entries
    seed: int

    @property
    def scale(self) -> float:
        # 1/sqrt(d) as the float32 the C-ABI receives
        return float(np.float32(1.0 / np.sqrt(self.d)))

    @property
    def label(self) -> str:
        return f"{self.B}x{self.H}x{self.N}x{self.d}"


# Small / Medium / Large / Large-with-backward / XL-with-backward.
WORKLOADS = {
    "c1": Workload("c1", 2, 8, 512, 64, (False,), False, 1.0, 1.0, 1),
    "c2": Workload("c2", 4, 32, 1024, 128, (True,), False, 1.0, 1.0, 2),
    "c3": Workload("c3", 8, 64, 2048, 128, (True, False), False, 1.0, 1.0, 3),
    "c4": Workload("c4", 8, 64, 2048, 128, (True,), True, 1.0, 1.0, 4),
    # large logits (Q, K ~ N(0, 3^2)) stress the running-max rescale
    "c5": Workload("c5", 4, 64, 4096, 128, (True,), True, 3.0, 1.0, 5),
}


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (round to nearest, ties to even).

    Returns the 16-bit patterns as uint16. NaNs stay NaN (quiet bit forced),
    infinities and signed zeros are preserved, subnormals round like any other
    value (bfloat16 keeps float32's exponent range).
    """
    x = np.ascontiguousarray(x, dtype=np.float32)
    u = x.view(np.uint32)
    lsb = (u >> np.uint32(16)) & np.uint32(1)
    rounded = (u + np.uint32(0x7FFF) + lsb) >> np.uint32(16)
    nan = np.isnan(x)
    out = rounded.astype(np.uint16)
    if nan.any():
        out[nan] = ((u[nan] >> np.uint32(16)) | np.uint32(0x0040)).astype(np.uint16)
    return out


def f32_to_f16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 values to IEEE binary16 (numpy's conversion: round to
    nearest, ties to even; overflow to infinity) and return the uint16 bits."""
    with np.errstate(over="ignore"):  # the overflow to infinity is the intended result
        return np.ascontiguousarray(x, dtype=np.float32).astype(np.float16).view(np.uint16)


def normal_bf16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """One tensor of N(0, sigma^2) samples rounded to bf16 (uint16 bits)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_bf16_bits(x)


def normal_f16(rng: np.random.Generator, shape, sigma: float) -> np.ndarray:
    """One tensor of N(0, sigma^2) samples rounded to binary16 (uint16 bits)."""
    x = rng.standard_normal(shape, dtype=np.float32)
    if sigma != 1.0:
        x *= np.float32(sigma)
    return f32_to_f16_bits(x)


def make_qkv(B: int, H: int, N: int, d: int, seed: int, *, sigma_qk: float = 1.0,
             sigma_v: float = 1.0, with_do: bool = False, dtype: str = "bf16",
             Hkv: int | None = None) -> dict:
    """Q, K, V (and dO) as 16-bit patterns: bf16 by default, IEEE binary16 with
    dtype="f16" (same draws, other rounding). Q and dO are [B, H, N, d]; K and
    V are [B, Hkv, N, d] (Hkv = H unless given)."""
    if dtype not in ("bf16", "f16"):
        raise ValueError(f"dtype must be 'bf16' or 'f16', got {dtype!r}")
    Hkv = H if Hkv is None else Hkv
    normal = normal_bf16 if dtype == "bf16" else normal_f16
    rng = np.random.default_rng(seed)
    shape = (B, H, N, d)
    kv_shape = (B, Hkv, N, d)
    out = {
        "q": normal(rng, shape, sigma_qk),
        "k": normal(rng, kv_shape, sigma_qk),
        "v": normal(rng, kv_shape, sigma_v),
    }
    if with_do:
        out["do"] = normal(rng, shape, sigma_v)
    return out


def make_inputs(w: Workload, seed: int | None = None) -> dict:
    """The inputs of one named workload (seeded with its own seed by default)."""
    return make_qkv(w.B, w.H, w.N, w.d, w.seed if seed is None else seed,
                    sigma_qk=w.sigma_qk, sigma_v=w.sigma_v, with_do=w.backward)
