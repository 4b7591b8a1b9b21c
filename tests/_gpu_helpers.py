"""Helpers for the GPU parity tests: moving tensors to the oracle and comparing.

Tolerance for attention (bf16 in, fp32 accumulate) against the float64 oracle, over
all compared output elements: max |gpu - oracle| <= 2e-2 and mean |gpu - oracle| <=
2e-3.  The store is compared bit for bit.
"""

from __future__ import annotations

import sys

import numpy as np
import torch

MAX_ABS = 2e-2
MEAN_ABS = 2e-3


def log(*a):
    print(*a, flush=True)
    sys.stdout.flush()


def elem(t: torch.Tensor) -> str:
    return "bf16" if t.dtype == torch.bfloat16 else "f32"


def host_bits(t: torch.Tensor) -> np.ndarray:
    """Raw element bits on the host: uint16 for bf16, float32 array for f32."""
    t = t.detach().contiguous().cpu()
    if t.dtype == torch.bfloat16:
        return t.view(torch.int16).numpy().view(np.uint16)
    return t.numpy()


def raw_bytes(t: torch.Tensor) -> np.ndarray:
    t = t.detach().contiguous().cpu()
    return t.view(torch.uint8).numpy() if t.dtype != torch.bfloat16 else \
        t.view(torch.int16).numpy().view(np.uint8)


def to_f64(t: torch.Tensor) -> np.ndarray:
    return t.detach().cpu().to(torch.float64).numpy()


def dev_i32(a, device) -> torch.Tensor:
    return torch.as_tensor(np.ascontiguousarray(a, dtype=np.int32), device=device)


def assert_close(got: np.ndarray, want: np.ndarray, what: str, max_abs=MAX_ABS, mean_abs=MEAN_ABS):
    assert got.shape == want.shape, (got.shape, want.shape)
    assert np.isfinite(want).all(), f"{what}: oracle produced non-finite values"
    assert np.isfinite(got).all(), f"{what}: kernel output has non-finite values"
    err = np.abs(got - want)
    mx, mean = float(err.max()), float(err.mean())
    log(f"  {what}: max_abs={mx:.3e} mean_abs={mean:.3e} n={err.size}")
    assert mx <= max_abs, f"{what}: max abs error {mx:.3e} > {max_abs}"
    assert mean <= mean_abs, f"{what}: mean abs error {mean:.3e} > {mean_abs}"
    return mx, mean


def require_gpu():
    if not torch.cuda.is_available():
        raise RuntimeError("GPU tests need a visible MI355X")
    return torch.device("cuda:0")
