"""Counter-seeded random tensors (see the package docstring)."""

from __future__ import annotations

import torch

WORKLOAD_SEED = 20261202

_MASK64 = (1 << 64) - 1


def _splitmix64(x: int) -> int:
    # Steele, Lea & Flood, "Fast splittable pseudorandom number generators"
    # (OOPSLA 2014): the splitmix64 finaliser.
    x = (x + 0x9E3779B97F4A7C15) & _MASK64
    x = ((x ^ (x >> 30)) * 0xBF58476D1CE4E5B9) & _MASK64
    x = ((x ^ (x >> 27)) * 0x94D049BB133111EB) & _MASK64
    return x ^ (x >> 31)


def seed_for(*keys: int) -> int:
    """A 63-bit seed from a tuple of integers (negative keys allowed)."""
    h = 0
    for k in keys:
        h = _splitmix64(h ^ (int(k) & _MASK64))
    return h & ((1 << 63) - 1)


def _gen(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal(n: int, std: float, seed: int, dtype=torch.float32, device="cpu") -> torch.Tensor:
    """n draws of N(0, std^2) (std is the standard deviation), cast to dtype."""
    g = _gen(seed, device)
    x = torch.randn(n, generator=g, device=device, dtype=torch.float32)
    x.mul_(std)
    return x.to(dtype)


def log_uniform_signed(n: int, lo: float, hi: float, seed: int, dtype=torch.float32,
                       device="cpu") -> torch.Tensor:
    """Magnitudes 10^U(log10 lo, log10 hi) with a random sign, cast to dtype."""
    import math

    g = _gen(seed, device)
    e = torch.empty(n, device=device, dtype=torch.float64)
    e.uniform_(math.log10(lo), math.log10(hi), generator=g)
    mag = torch.pow(10.0, e)
    sign = torch.randint(0, 2, (n,), generator=g, device=device, dtype=torch.int8)
    mag = torch.where(sign.bool(), -mag, mag)
    return mag.to(dtype)


def shared_mask(n: int, frac: float, seed: int, device="cpu") -> torch.Tensor:
    """Bool mask with each position set with probability frac."""
    g = _gen(seed, device)
    u = torch.rand(n, generator=g, device=device, dtype=torch.float32)
    return u < frac


def fill_pattern(t: torch.Tensor, value_bits: int) -> torch.Tensor:
    """Fill a 16- or 32-bit tensor with one raw bit pattern (canary value)."""
    if t.element_size() == 2:
        t.view(torch.int16).fill_(value_bits - (1 << 16) if value_bits >= 1 << 15 else value_bits)
    elif t.element_size() == 4:
        t.view(torch.int32).fill_(value_bits - (1 << 32) if value_bits >= 1 << 31 else value_bits)
    else:
        raise ValueError("fill_pattern: 2- or 4-byte elements only")
    return t
