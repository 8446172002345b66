"""Helpers for GPU tests: moving bf16 bit patterns to the device and back, and
the error measures the acceptance bars are written in."""
from __future__ import annotations

import numpy as np

# Acceptance bars for bf16 inputs with float32 accumulation:
O_ATOL = 2e-2       # max |O_gpu - O_ref|
LSE_ATOL = 2e-2     # max |LSE_gpu - LSE_ref|
GRAD_RTOL = 5e-2    # max |X_gpu - X_ref| / max |X_ref|, X in dQ, dK, dV


def to_dev(bits: np.ndarray, device="cuda"):
    import torch
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def to_f64(t) -> np.ndarray:
    import torch
    return t.detach().to("cpu", torch.float64).numpy()


def max_abs(a, b) -> float:
    return float(np.max(np.abs(np.asarray(a, np.float64) - np.asarray(b, np.float64))))


def rel_to_max(a, b) -> float:
    den = float(np.max(np.abs(b)))
    return max_abs(a, b) / den if den > 0 else max_abs(a, b)


def announce(msg: str):
    print(msg, flush=True)
