"""Helpers for the GPU parity tests: host <-> device copies of generated inputs."""

from __future__ import annotations

import sys

import numpy as np
import torch

DEV = "cuda:0"


def say(msg: str) -> None:
    """Print and flush a progress line (names the case before each GPU step)."""
    print(msg, flush=True)
    sys.stdout.flush()


def to_dev(t) -> torch.Tensor:
    """A synth.Tensor (or float32 / int array) -> a device tensor of the stored dtype."""
    if hasattr(t, "bits"):
        if t.bits is not None:
            return torch.from_numpy(np.ascontiguousarray(t.bits).view(np.int16)).to(DEV).view(
                torch.bfloat16)
        return torch.from_numpy(np.ascontiguousarray(t.f32)).to(DEV)
    a = np.ascontiguousarray(t)
    return torch.from_numpy(a).to(DEV)


def from_dev(x: torch.Tensor) -> np.ndarray:
    """Device tensor -> float64 (for bf16/fp32) or the integer array."""
    x = x.detach().cpu()
    if x.dtype == torch.bfloat16:
        return x.float().numpy().astype(np.float64)
    if x.dtype == torch.float32:
        return x.numpy().astype(np.float64)
    return x.numpy()


def bf16_bits(x: torch.Tensor) -> np.ndarray:
    return x.detach().cpu().view(torch.int16).numpy().view(np.uint16)


def max_abs(a, b) -> float:
    """Max |a - b|; +inf if either side holds a NaN or Inf (never silently dropped)."""
    a = np.asarray(a, np.float64)
    b = np.asarray(b, np.float64)
    if not (np.isfinite(a).all() and np.isfinite(b).all()):
        return float("inf")
    return float(np.max(np.abs(a - b))) if a.size else 0.0
