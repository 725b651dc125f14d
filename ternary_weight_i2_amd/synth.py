"""Seeded synthetic inputs for the W2A8 (I2_S) matmul workloads.

This module only draws random numbers: ternary weight matrices, per-tensor
weight scales and activation tokens.  It holds none of the method's arithmetic
(no packing, no quantisation, no dot) so that both the GPU library's tests and
the CPU oracle can consume the same inputs without sharing code.

Every draw is keyed by ``numpy.random.SeedSequence([base, workload, layer,
proj, role])`` so any single matrix or token block can be regenerated alone.

Workloads (shapes as M x K = output rows x reduction length):

* ``single``  -- one 256x512 matrix, uniform ternary, one fp32 token.
* ``b2``      -- 2B-class layer (hidden 2560, FFN 6912, 20 query heads and 5
  KV heads of dim 128): q/o 2560x2560, k/v 640x2560, gate/up 6912x2560,
  down 2560x6912; uniform ternary; bf16 tokens.
* ``b2_sparse`` -- the same shapes with p(0)=1/2, p(+1)=p(-1)=1/4 and bf16
  tokens where odd token rows carry one +-20 outlier (20 sigma); a single
  token is run both plain and with one (``outliers="all"``).
* ``e06``     -- 0.6B-class embedding model (hidden 1024, FFN 3072, 16 query
  heads of dim 128, 8 KV heads): q 2048x1024, k/v 1024x1024, o 1024x2048,
  gate/up 3072x1024, down 1024x3072; uniform ternary; bf16 tokens.
* ``large``   -- hidden 8192, FFN 28672, 64 query / 8 KV heads of dim 128:
  q/o 8192x8192, k/v 1024x8192, gate/up 28672x8192, down 8192x28672, 8
  layers; uniform ternary; bf16 tokens.
"""
from __future__ import annotations

import numpy as np

BASE_SEED = 20251

WORKLOAD_IDS = {"single": 1, "b2": 2, "b2_sparse": 3, "e06": 4, "large": 5}
ROLE_IDS = {"weights": 0, "act": 1, "scale": 2, "outlier": 3}
PROJ_NAMES = ("q", "k", "v", "o", "gate", "up", "down")

SHAPES = {
    "single": {"w": (256, 512)},
    "b2": {"q": (2560, 2560), "k": (640, 2560), "v": (640, 2560),
           "o": (2560, 2560), "gate": (6912, 2560), "up": (6912, 2560),
           "down": (2560, 6912)},
    "e06": {"q": (2048, 1024), "k": (1024, 1024), "v": (1024, 1024),
            "o": (1024, 2048), "gate": (3072, 1024), "up": (3072, 1024),
            "down": (1024, 3072)},
    "large": {"q": (8192, 8192), "k": (1024, 8192), "v": (1024, 8192),
              "o": (8192, 8192), "gate": (28672, 8192), "up": (28672, 8192),
              "down": (8192, 28672)},
}
SHAPES["b2_sparse"] = SHAPES["b2"]
LAYERS = {"single": 1, "b2": 30, "b2_sparse": 1, "e06": 1, "large": 8}
TOKENS = {"single": (1,), "b2": (1,), "b2_sparse": (1, 4, 16, 64),
          "e06": (128, 4096), "large": (1, 16)}


def rng_for(workload: str, layer: int = 0, proj: str | int = 0,
            role: str = "weights") -> np.random.Generator:
    p = PROJ_NAMES.index(proj) if isinstance(proj, str) and proj in PROJ_NAMES else (
        0 if isinstance(proj, str) else int(proj))
    ss = np.random.SeedSequence([BASE_SEED, WORKLOAD_IDS[workload], int(layer),
                                 int(p), ROLE_IDS[role]])
    return np.random.default_rng(ss)


def ternary(rng: np.random.Generator, M: int, K: int,
            dist: str = "uniform") -> np.ndarray:
    """int8 [M][K] with entries in {-1, 0, +1}.

    ``uniform``: each value with probability 1/3.  ``half_zero``: 0 with
    probability 1/2, +1 and -1 with 1/4 each.
    """
    if dist == "uniform":
        return (rng.integers(0, 3, size=(M, K), dtype=np.int8) - 1).astype(np.int8)
    if dist == "half_zero":
        u = rng.integers(0, 4, size=(M, K), dtype=np.int8)
        out = np.zeros((M, K), dtype=np.int8)
        out[u == 2] = 1
        out[u == 3] = -1
        return out
    raise ValueError(dist)


def weight_scale(rng: np.random.Generator) -> float:
    """Per-tensor fp32 weight scale drawn uniform in [0.01, 0.1]."""
    return float(np.float32(rng.uniform(0.01, 0.1)))


def f32_to_bf16_bits(x: np.ndarray) -> np.ndarray:
    """Round float32 samples to bf16 (nearest, ties to even); returns uint16 bits."""
    b = np.ascontiguousarray(x, dtype=np.float32).view(np.uint32).astype(np.uint64)
    r = (b + 0x7FFF + ((b >> 16) & 1)) >> 16
    return r.astype(np.uint16)


def bf16_bits_to_f32(h: np.ndarray) -> np.ndarray:
    return (np.ascontiguousarray(h, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def tokens_f32(rng: np.random.Generator, N: int, K: int) -> np.ndarray:
    """fp32 [N][K] ~ N(0, 1)."""
    return rng.standard_normal((N, K), dtype=np.float32)


def tokens_bf16(rng: np.random.Generator, N: int, K: int,
                outliers: bool | str = False,
                orng: np.random.Generator | None = None) -> np.ndarray:
    """bf16 bits [N][K]: N(0,1) samples rounded to bf16.  With ``outliers``
    (True or "odd"), every odd token row gets one element (seeded position and
    sign) set to +-20.0, which is exact in bf16; with "all", every row does
    (so a single token carries one too)."""
    x = tokens_f32(rng, N, K)
    if outliers:
        if outliers not in (True, "odd", "all"):
            raise ValueError(outliers)
        orng = orng or rng
        for n in range(0 if outliers == "all" else 1, N, 1 if outliers == "all" else 2):
            k = int(orng.integers(0, K))
            x[n, k] = np.float32(20.0 if orng.integers(0, 2) else -20.0)
    return f32_to_bf16_bits(x)


def matrix(workload: str, proj: str, layer: int = 0):
    """(int8 ternary W, fp32 alpha) of one projection of one layer."""
    M, K = SHAPES[workload][proj]
    dist = "half_zero" if workload == "b2_sparse" else "uniform"
    W = ternary(rng_for(workload, layer, proj, "weights"), M, K, dist)
    alpha = weight_scale(rng_for(workload, layer, proj, "scale"))
    return W, alpha


def activations(workload: str, proj: str, N: int, layer: int = 0) -> np.ndarray:
    """Tokens for one projection: fp32 for ``single``, bf16 bits otherwise."""
    K = SHAPES[workload][proj][1]
    r = rng_for(workload, layer, proj, "act")
    if workload == "single":
        return tokens_f32(r, N, K)
    return tokens_bf16(r, N, K, outliers=(workload == "b2_sparse"),
                       orng=rng_for(workload, layer, proj, "outlier"))


# ---- device-side draws for large benchmark stacks ---------------------------
# Hundreds of MB of weights are drawn directly on the GPU with torch's seeded
# generator (no arithmetic of the method involved); tests draw on the host.

def ternary_torch(M: int, K: int, seed: int, device="cuda", dist: str = "uniform"):
    """int8 [M][K] ternary tensor drawn on ``device`` with a seeded generator."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    if dist == "uniform":
        return torch.randint(0, 3, (M, K), dtype=torch.int8, device=device, generator=g) - 1
    if dist == "half_zero":
        u = torch.randint(0, 4, (M, K), dtype=torch.int8, device=device, generator=g)
        out = torch.zeros((M, K), dtype=torch.int8, device=device)
        out[u == 2] = 1
        out[u == 3] = -1
        return out
    raise ValueError(dist)


def tokens_bf16_torch(N: int, K: int, seed: int, device="cuda"):
    """bf16 [N][K] ~ N(0,1) drawn on ``device`` (fp32 sample rounded to bf16)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(int(seed))
    return torch.randn((N, K), dtype=torch.float32, device=device, generator=g).to(torch.bfloat16)


def stack_seed(workload: str, layer: int, proj: str, role: str) -> int:
    """A 63-bit seed for device-side draws, derived like ``rng_for``."""
    return int(rng_for(workload, layer, proj, role).integers(0, 2 ** 63 - 1))
