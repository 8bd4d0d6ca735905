"""Seeded synthetic inputs shared by the tests, the benchmark and the smoke check.

This module holds no part of the W12 method: it draws Gaussian weights and
activations, rounds them to BF16 and sprinkles exact zeros.  Bringing raw
weights into a group's encodable exponent range is format arithmetic and is
done by the callers (through a pack/unpack round trip), not here.

The workloads stand in for the checkpoints of the 8-30B dense models the
pages measure on (AI Radar summary of SpecPilot, English edition, "Reasons":
8-30B dense models; HotRepo digest of StargazerX0/SpecPilot, project
introduction: batch 1-32), which are not available: shapes are those of the
linear layers of a ~27B dense decoder, values are N(0, sigma) draws.

Recipe (numpy PCG64 via ``default_rng``):
  * weights: fp32 standard normal * sigma, rounded to BF16 (round to nearest
    even), then a Bernoulli(p_zero) mask drawn from its own seed replaces an
    element by a zero that keeps the drawn sign (so +0 and -0 both occur);
  * activations: fp32 standard normal * sigma_x, rounded to BF16.

The 64-layer stack (21.1 billion weights) is drawn by the same recipe on the
device instead (``device_weights``: torch's seeded Philox generator), since
drawing it on the host takes minutes; it only feeds throughput figures.
"""
from __future__ import annotations

from dataclasses import dataclass

import numpy as np


def f32_to_bf16_bits(a: np.ndarray) -> np.ndarray:
    """Round fp32 to the nearest BF16 (ties to even); NaN stays a quiet NaN."""
    a = np.ascontiguousarray(a, dtype=np.float32)
    u = a.view(np.uint32)
    # no uint32 overflow: the largest non-NaN pattern 0xFF800000 + 0x8000 fits
    rounded = ((u + np.uint32(0x7FFF) + ((u >> 16) & np.uint32(1))) >> 16).astype(np.uint16)
    nan = np.isnan(a)
    if nan.any():
        rounded[nan] = ((u[nan] >> 16).astype(np.uint16) | np.uint16(0x0040))
    return rounded


def bf16_bits_to_f32(a: np.ndarray) -> np.ndarray:
    a = np.asarray(a, dtype=np.uint16)
    return (a.astype(np.uint32) << 16).view(np.float32)


def gaussian_bf16(shape, sigma: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    a = rng.standard_normal(shape, dtype=np.float32)
    a *= np.float32(sigma)
    return f32_to_bf16_bits(a)


def inject_zeros(w: np.ndarray, p_zero: float, seed: int) -> np.ndarray:
    """Replace a Bernoulli(p_zero) subset by signed zeros (sign of the draw)."""
    rng = np.random.default_rng(seed)
    mask = rng.random(w.shape, dtype=np.float32) < np.float32(p_zero)
    out = w.copy()
    out[mask] &= np.uint16(0x8000)
    return out


@dataclass(frozen=True)
class GemmCase:
    """One GEMM workload: W [N, K] ~ N(0, sigma_w), x [M, K] ~ N(0, sigma_x)."""
    name: str
    N: int
    K: int
    M: int
    sigma_w: float
    sigma_x: float
    seed_w: int
    seed_x: int
    seed_zero: int
    p_zero: float = 0.001

    def weights_raw(self) -> np.ndarray:
        w = gaussian_bf16((self.N, self.K), self.sigma_w, self.seed_w)
        return inject_zeros(w, self.p_zero, self.seed_zero)

    def activations(self, M: int | None = None) -> np.ndarray:
        M = self.M if M is None else M
        return gaussian_bf16((M, self.K), self.sigma_x, self.seed_x + 1000 * M)

    @property
    def weight_elems(self) -> int:
        return self.N * self.K


# The five workloads: a tiny case, then linear layers of a ~27B dense decoder
# (hidden 5120, QKV out 7168, fused gate+up 34816, down in 17408).
TINY = GemmCase("tiny 1024x512", 1024, 512, 1, 0.02, 1.0, 101, 102, 103)
QKV = GemmCase("qkv 7168x5120", 7168, 5120, 1, 0.02, 1.0, 201, 202, 203)
GATE_UP = GemmCase("gate_up 34816x5120", 34816, 5120, 16, 0.02, 1.0, 301, 302, 303)
DOWN = GemmCase("down 5120x17408", 5120, 17408, 32, 0.015, 0.5, 401, 402, 403)
# the attention output projection of the same decoder (part of the stack)
O_PROJ = GemmCase("o 5120x5120", 5120, 5120, 1, 0.02, 1.0, 501, 502, 503)

CASES = {c.name.split()[0]: c for c in (TINY, QKV, GATE_UP, DOWN, O_PROJ)}

# One GPU's share of the same four weights under 8-way tensor parallelism:
# QKV and gate+up split along N (their output rows), O and down along K.
SHARD_CASES = {c.name.split()[0]: c for c in (
    GemmCase("qkv_tp8 896x5120", 896, 5120, 1, 0.02, 1.0, 601, 602, 603),
    GemmCase("o_tp8 5120x640", 5120, 640, 1, 0.02, 1.0, 611, 612, 613),
    GemmCase("gate_up_tp8 4352x5120", 4352, 5120, 1, 0.02, 1.0, 621, 622, 623),
    GemmCase("down_tp8 5120x2176", 5120, 2176, 1, 0.015, 0.5, 631, 632, 633))}

# 64-layer stack: per layer QKV, O, gate+up, down (N, K).
STACK_LAYERS = 64
STACK_SHAPES = ((7168, 5120), (5120, 5120), (34816, 5120), (5120, 17408))


def device_weights(torch, N: int, K: int, seed: int, sigma: float = 0.02,
                   p_zero: float = 0.001):
    """The weight recipe drawn on the current GPU with a seeded torch
    generator: fp32 N(0, sigma) -> BF16 (torch rounds to nearest even), then a
    Bernoulli(p_zero) subset set to zero with the drawn sign."""
    g = torch.Generator(device="cuda")
    g.manual_seed(seed)
    w = torch.randn((N, K), generator=g, device="cuda", dtype=torch.float32)
    w.mul_(sigma)
    zero = torch.rand((N, K), generator=g, device="cuda") < p_zero
    w = w.to(torch.bfloat16)
    bits = w.view(torch.int16)
    bits[zero] &= -0x8000                # keep only the sign bit
    return w
