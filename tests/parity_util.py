"""Helpers for GPU-vs-oracle parity tests: exact value transfer and tolerances."""

import numpy as np
import torch

import oracle

# Relative Frobenius error of the GPU projection against the float64 oracle:
# 5e-3 for bf16 inputs with fp32 accumulation, 1e-5 for fp32 inputs.
BF16_TOL = 5e-3
F32_TOL = 1e-5


def bits_to_device(bits: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(bits).view(np.int16)).view(torch.bfloat16).to(device)


def f32_to_device(a: np.ndarray, device="cuda") -> torch.Tensor:
    return torch.from_numpy(np.ascontiguousarray(a, dtype=np.float32)).to(device)


def exact(t: torch.Tensor) -> np.ndarray:
    """Exact float64 values of a bf16 or fp32 tensor (any device)."""
    t = t.detach().cpu().contiguous()
    if t.dtype == torch.bfloat16:
        return oracle.bf16_bits_to_f64(t.view(torch.int16).numpy().view(np.uint16))
    if t.dtype == torch.float32:
        return t.numpy().astype(np.float64)
    if t.dtype == torch.float64:
        return t.numpy().copy()
    raise TypeError(t.dtype)


def tol_for(dtype) -> float:
    return BF16_TOL if dtype == torch.bfloat16 else F32_TOL


def sample_rows(n: int, k: int, seed: int) -> np.ndarray:
    """k distinct indices in [0, n) including the first and last (sorted)."""
    if n <= k:
        return np.arange(n)
    r = np.random.default_rng(seed)
    pick = set(r.choice(n, size=k - 2, replace=False).tolist()) | {0, n - 1}
    return np.array(sorted(pick))
