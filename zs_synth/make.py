"""Tensor builders for the workloads (random draws only; see the package docstring)."""

from __future__ import annotations

import torch

from .gen import WORKLOAD_SEED, seed_for, normal, log_uniform_signed, shared_mask
from .workloads import Workload, const_value

TORCH_DTYPE = {"f16": torch.float16, "bf16": torch.bfloat16, "f32": torch.float32}

# stream ids inside a (rank, step) seed
_S_GRAD, _S_W0, _S_MASK, _S_STATE = 1, 2, 3, 4


def initial_w(wl: Workload, k: int, length: int, device="cpu") -> torch.Tensor:
    """fp32 master weights of shard k at step 0, ~N(0, w_std^2)."""
    return normal(length, wl.w_std, seed_for(WORKLOAD_SEED, -1, 0, _S_W0, k), torch.float32,
                  device)


def normal_grad(wl: Workload, rank: int, step: int, length: int, device="cpu",
                stream: int = 0) -> torch.Tensor:
    """Rank `rank`'s local gradient at 1-based step `step`, ~N(0, grad_std^2),
    rounded to the gradient dtype.  `stream` separates independent buffers
    (e.g. one per shard when every shard has its own slice buffers)."""
    return normal(length, wl.grad_std, seed_for(WORKLOAD_SEED, rank, step, _S_GRAD, stream),
                  TORCH_DTYPE[wl.grad_dtype], device)


def edge_zero_mask(wl: Workload, n: int, device="cpu") -> torch.Tensor:
    """Positions whose gradient is exactly zero on every rank and every step."""
    return shared_mask(n, wl.zero_frac, seed_for(WORKLOAD_SEED, -2, 0, _S_MASK), device)


def edge_grad(wl: Workload, rank: int, step: int, n: int, zero_mask: torch.Tensor,
              shard_starts, shard_ends, device="cpu") -> torch.Tensor:
    """Full-length edge gradient of one rank: magnitudes 10^U(log lo, log hi)
    with a random sign, exact zeros where zero_mask is set, and for every shard
    k a block of const_block positions from shard_starts[k] holding
    const_value(k) on all ranks and steps."""
    x = log_uniform_signed(n, wl.edge_lo, wl.edge_hi,
                           seed_for(WORKLOAD_SEED, rank, step, _S_GRAD), torch.float32, device)
    x.masked_fill_(zero_mask, 0.0)
    for k, (s, e) in enumerate(zip(shard_starts, shard_ends)):
        b = min(wl.const_block, e - s)
        if b > 0:
            x[s:s + b] = const_value(k)
    return x.to(TORCH_DTYPE[wl.grad_dtype])


def random_state(length: int, seed_key: int, device="cpu"):
    """(m, v) with m ~ N(0, 1e-3^2) and v = |N(0, 1e-6^2)| for tests that start
    from a mid-training state instead of m0 = v0 = 0."""
    m = normal(length, 1e-3, seed_for(WORKLOAD_SEED, -3, seed_key, _S_STATE, 0), torch.float32,
               device)
    v = normal(length, 1e-6, seed_for(WORKLOAD_SEED, -3, seed_key, _S_STATE, 1), torch.float32,
               device).abs_()
    return m, v
