"""Seeded synthetic inputs for the fused FP8 LayerNorm modules.

This module only draws random numbers and rounds them to bf16.  It holds no
step of the method itself (no LayerNorm, no scaling, no FP8 encoding), so both
the HIP path's callers and the CPU oracle may take their inputs from it.

Workload shapes follow the GPT-style model of the Transformer Engine tutorial
("Accelerating Transformer Training with NVIDIA Transformer Engine, Fused
Kernels, BF16, FP8, and GPU Benchmarking", model and benchmark listings):
hidden 768, FFN 3072, sequence 256, batch 8 (module tour) and 32 (benchmark),
plus the scale-up to hidden 2048 suggested in its closing "things to try"
list.  Values are N(0, 1) activations, N(0, 0.02) weights, LayerNorm gains
1 + 0.1 N(0, 1) and shifts 0.1 N(0, 1).

Every tensor gets its own seed, derived from the tutorial's base seed 1234,
a workload name, a tensor name and a step index, so any tensor can be
regenerated alone.  Numbers come from torch's Philox generator on the
requested device; a test that compares two implementations draws once and
hands the same bytes to both.
"""
from __future__ import annotations

import zlib

import torch

BASE_SEED = 1234


def seed_for(workload: str, tensor: str, step: int = 0) -> int:
    """Deterministic 63-bit seed for one tensor of one step of one workload."""
    key = f"{BASE_SEED}/{workload}/{tensor}/{step}".encode()
    hi = zlib.crc32(key)
    lo = zlib.crc32(key[::-1])
    return ((hi << 32) | lo) & 0x7FFF_FFFF_FFFF_FFFF


def _generator(seed: int, device) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def normal_bf16(shape, seed: int, std: float = 1.0, mean: float = 0.0,
                device="cpu") -> torch.Tensor:
    """mean + std * N(0, 1), drawn in fp32 and rounded to bf16 (nearest-even)."""
    g = _generator(seed, device)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    if std != 1.0:
        t.mul_(std)
    if mean != 0.0:
        t.add_(mean)
    return t.to(torch.bfloat16)


def spiky_normal_bf16(shape, seed: int, drift: float = 1.0, spike_prob: float = 1e-3,
                      spike_factor: float = 100.0, device="cpu") -> torch.Tensor:
    """drift * N(0, 1) with a Bernoulli(spike_prob) mask of entries scaled by
    spike_factor, applied in fp32 before the bf16 rounding."""
    g = _generator(seed, device)
    t = torch.randn(tuple(shape), generator=g, dtype=torch.float32, device=device)
    u = torch.rand(tuple(shape), generator=g, dtype=torch.float32, device=device)
    t.mul_(drift)
    t = torch.where(u < spike_prob, t * spike_factor, t)
    return t.to(torch.bfloat16)


def layernorm_params(hidden: int, workload: str, device="cpu"):
    """gamma = 1 + 0.1 N(0, 1), beta = 0.1 N(0, 1), both bf16 [hidden]."""
    gamma = normal_bf16((hidden,), seed_for(workload, "gamma"), std=0.1, mean=1.0,
                        device=device)
    beta = normal_bf16((hidden,), seed_for(workload, "beta"), std=0.1, device=device)
    return gamma, beta


def linear_weight(out_features: int, in_features: int, workload: str, name: str,
                  device="cpu") -> torch.Tensor:
    """N(0, 0.02) bf16 weight in [out][in] layout (torch.nn.Linear's layout)."""
    return normal_bf16((out_features, in_features), seed_for(workload, name), std=0.02,
                       device=device)


def drift_factor(step: int, n_steps: int, start: float = 1.0, end: float = 4.0) -> float:
    """Linear input-scale drift from start (first step) to end (last step)."""
    if n_steps <= 1:
        return start
    return start + (end - start) * step / (n_steps - 1)


def random_history(length: int, n_slots: int, seed: int, device="cpu") -> torch.Tensor:
    """A positive fp32 amax history [length][n_slots] spanning many binades
    (log-uniform between 2^-20 and 2^20), for exercising the scale update."""
    g = _generator(seed, device)
    e = torch.rand((length, n_slots), generator=g, dtype=torch.float64, device=device)
    return torch.exp2(e * 40.0 - 20.0).to(torch.float32)
