"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle.

This module only draws random tensors and describes layer shapes; it holds no
quantisation, dequantisation or matmul arithmetic.  The same tensor (as BF16
bits) is handed to the HIP library and to the CPU oracle.

Recipe (all draws in float32, then rounded to BF16 by torch's conversion):
* W [N][K] ~ N(0, 0.02); a set S of round(0.01 K) "salient" input channels is
  multiplied by 8.  Salient channels are 0.1-1% of channels, picked out by
  activation magnitude (cyankiwi Quantization docs, "The Baseline: AWQ";
  Weight-Only Quantization and Mixed Precision, "3. AWQ").
* Optional per-group mean shift: W[n, 128g:128g+128] += mu[n,g],
  mu ~ U(-0.01, 0.01), applied after the salient scaling, so that zero points
  move away from the middle of the code range.
* X [M][K] ~ N(0, 1) with the same channel set S multiplied by 20 (the
  activation outliers that make those weight channels salient).
* Calibration activations for the AWQ importance use the X recipe with their
  own seed.

Seeds are a fixed function of (config id, layer name, tensor role, M).
"""

from __future__ import annotations

import hashlib
from dataclasses import dataclass

import torch

BASE_SEED = 20261203
GROUP = 128


def seed_of(*parts) -> int:
    """Deterministic 63-bit seed from any tuple of ints/strings."""
    h = hashlib.sha256(repr((BASE_SEED,) + tuple(parts)).encode()).digest()
    return int.from_bytes(h[:8], "little") & ((1 << 63) - 1)


def _gen(device, seed: int) -> torch.Generator:
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    return g


def salient_channels(K: int, cfg, layer: str) -> torch.Tensor:
    """round(0.01 K) distinct channel indices (CPU int64), shared by a layer's
    W and X."""
    n = int(round(0.01 * K))
    g = _gen("cpu", seed_of(cfg, layer, "salient"))
    return torch.randperm(K, generator=g)[:n].sort().values


def weights(N: int, K: int, cfg, layer: str, *, shift: bool = False,
            device="cpu") -> torch.Tensor:
    """BF16 weight matrix [N][K] on `device` (see module recipe)."""
    g = _gen(device, seed_of(cfg, layer, "W"))
    w = torch.randn(N, K, generator=g, device=device, dtype=torch.float32)
    w.mul_(0.02)
    S = salient_channels(K, cfg, layer).to(device)
    w[:, S] *= 8.0
    if shift:
        assert K % GROUP == 0
        gm = _gen(device, seed_of(cfg, layer, "mu"))
        mu = torch.rand(N, K // GROUP, generator=gm, device=device, dtype=torch.float32)
        mu.mul_(0.02).sub_(0.01)
        w.view(N, K // GROUP, GROUP).add_(mu.unsqueeze(-1))
        del mu
    out = w.to(torch.bfloat16)
    del w
    return out


def activations(M: int, K: int, cfg, layer: str, *, role: str = "X",
                device="cpu") -> torch.Tensor:
    """BF16 activations [M][K] ~ N(0,1), salient channels x20."""
    g = _gen(device, seed_of(cfg, layer, role, M))
    x = torch.randn(M, K, generator=g, device=device, dtype=torch.float32)
    S = salient_channels(K, cfg, layer).to(device)
    x[:, S] *= 20.0
    return x.to(torch.bfloat16)


def hand_groups() -> dict:
    """Constructed 128-value groups (float64 values, exactly representable in
    BF16), the special cases of the quantiser: a constant group and its
    negation, an all-zero group, a subnormal constant, alternating +-2^-125
    (its scale is the smallest normal BF16 value), values on a grid far
    from zero (large negative zero point), and an exact grid of step 2^-7."""
    import numpy as np
    j = np.arange(GROUP) % 16
    return {
        "const": np.full(GROUP, 0.375),
        "neg_const": np.full(GROUP, -0.375),
        "zero": np.zeros(GROUP),
        "subnormal_const": np.full(GROUP, 2.0 ** -130),
        "pm_2^-125": np.where(np.arange(GROUP) % 2 == 0, -(2.0 ** -125), 2.0 ** -125),
        "far_from_zero": 100.0 + 0.5 * (np.arange(GROUP) % 8),
        "grid_2^-7": (j - 8) * 2.0 ** -7,
    }


def extreme_weights(N: int, K: int, cfg, layer: str, *, device="cpu") -> torch.Tensor:
    """BF16 weights [N][K] whose groups of 128 are either ordinary draws
    (N(0, 0.02) or N(0, 1)) or one of hand_groups(), in a seeded random
    order per row, so that tiny, zero and huge group scales follow ordinary
    ones in every combination.  Even rows take no all-zero or subnormal
    group (groups whose weights are all zero); odd rows take every kind."""
    import numpy as np
    assert K % GROUP == 0
    G = K // GROUP
    names = list(hand_groups())
    hand = list(hand_groups().values())
    rng = np.random.default_rng(seed_of(cfg, layer, "extreme") & 0xFFFFFFFF)
    kind = rng.integers(0, 2 + len(hand), size=(N, G))
    nonzero = [2 + i for i, n in enumerate(names) if n not in ("zero", "subnormal_const")]
    pool = np.array([0, 1] + nonzero)
    even = rng.integers(0, len(pool), size=(N, G))
    kind[0::2] = pool[even[0::2]]
    w = np.empty((N, K), dtype=np.float64)
    ordinary = rng.standard_normal((N, K))
    for n in range(N):
        for g in range(G):
            c = kind[n, g]
            seg = slice(g * GROUP, (g + 1) * GROUP)
            if c == 0:
                w[n, seg] = 0.02 * ordinary[n, seg]
            elif c == 1:
                w[n, seg] = ordinary[n, seg]
            else:
                w[n, seg] = hand[c - 2]
    t = torch.from_numpy(w.astype(np.float32)).to(torch.bfloat16)
    return t.to(device)


def channel_vector(K: int, cfg, layer: str, role: str, *, device="cpu") -> torch.Tensor:
    """A positive float32 per-channel vector exp(N(0, 0.5^2)), used as an
    arbitrary AWQ pre-scale when testing the packer on its own."""
    g = _gen(device, seed_of(cfg, layer, role))
    v = torch.randn(K, generator=g, device=device, dtype=torch.float32)
    return torch.exp(0.5 * v)


def bits(t: torch.Tensor):
    """BF16 tensor -> numpy uint16 bit patterns (CPU copy)."""
    assert t.dtype == torch.bfloat16
    return t.detach().cpu().contiguous().view(torch.int16).numpy().view("uint16")


def from_bits(b, device="cpu") -> torch.Tensor:
    """numpy uint16 bit patterns -> BF16 tensor."""
    import numpy as np
    a = np.ascontiguousarray(b, dtype=np.uint16)
    return torch.from_numpy(a.view(np.int16).copy()).view(torch.bfloat16).to(device)


# ---------------------------------------------------------------------------
# Layer shapes of the synthetic workloads
# ---------------------------------------------------------------------------

@dataclass(frozen=True)
class Layer:
    name: str
    N: int   # output features
    K: int   # input features


# One 4096 x 4096 linear.
SINGLE_4096 = [Layer("linear", 4096, 4096)]

# Llama-3-8B-shaped decoder linears (hidden 4096, 32 q / 8 kv heads of 128,
# SwiGLU intermediate 14336).
LLAMA8B = [
    Layer("qkv", 6144, 4096),
    Layer("o", 4096, 4096),
    Layer("gate_up", 28672, 4096),
    Layer("down", 4096, 14336),
]

# 70B-shaped decoder linears (hidden 8192, 64 q / 8 kv heads, intermediate 28672).
LLAMA70B = [
    Layer("qkv", 10240, 8192),
    Layer("o", 8192, 8192),
    Layer("gate_up", 57344, 8192),
    Layer("down", 8192, 28672),
]

# One layer of the 40-layer stack: hidden 5120, 40 q / 8 kv heads of 128,
# SwiGLU intermediate 27648.
STACK40_LAYER = [
    Layer("qkv", 7168, 5120),
    Layer("o", 5120, 5120),
    Layer("gate_up", 55296, 5120),
    Layer("down", 5120, 27648),
]
STACK40_DEPTH = 40

WORKLOADS = {
    "single_4096": dict(layers=SINGLE_4096, Ms=[1], shift=False),
    "llama8b_decode": dict(layers=LLAMA8B, Ms=[1, 4, 8, 16, 32], shift=False),
    "llama70b_decode": dict(layers=LLAMA70B, Ms=[1, 8, 32], shift=True),
    "llama8b_prefill": dict(layers=LLAMA8B, Ms=[512, 2048, 4096], shift=False),
    "stack40_decode": dict(layers=STACK40_LAYER, Ms=[1, 8], shift=False,
                           depth=STACK40_DEPTH, awq_alpha=0.5, calib_tokens=512),
}
