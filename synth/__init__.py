"""Seeded synthetic inputs for the BitLinear layer.

This module draws random numbers and knows the layer shapes of the model
classes the pages discuss (a 2B model, a 3B model, a 70B model).  It holds
none of the layer's arithmetic: no scale, no rounding, no packing.  Both the
CPU oracle's tests and the HIP path's tests and benchmark take their inputs
from here, and nothing else is shared between the two.

Shapes are (name, K, N) with K = input features and N = output features;
weights are N x K fp32 row-major, activations M x K fp32 row-major.
"""
from __future__ import annotations

import numpy as np

# BitNet-class layer shapes.  The pages name the model sizes (a 2B model
# trained on 4T tokens; 3B and 70B cost points in the anthology note); the
# hidden/FFN sizes below are the standard ones for those classes.
SHAPES_2B = [("q", 2560, 2560), ("k", 2560, 640), ("v", 2560, 640), ("o", 2560, 2560),
             ("gate", 2560, 6912), ("up", 2560, 6912), ("down", 6912, 2560)]
SHAPES_3B = [("q", 3200, 3200), ("k", 3200, 3200), ("v", 3200, 3200), ("o", 3200, 3200),
             ("gate", 3200, 8640), ("up", 3200, 8640), ("down", 8640, 3200)]
SHAPES_70B = [("q", 8192, 8192), ("k", 8192, 1024), ("v", 8192, 1024), ("o", 8192, 8192),
              ("gate", 8192, 28672), ("up", 8192, 28672), ("down", 28672, 8192)]

MODELS = {
    "2b": {"shapes": SHAPES_2B, "layers": 30, "sigma": 0.02},
    "3b": {"shapes": SHAPES_3B, "layers": 26, "sigma": 0.02},
    "70b": {"shapes": SHAPES_70B, "layers": 80, "sigma": 0.01},
}


def matrix_seed(layer: int, j: int) -> int:
    """Seed of the j-th matrix (q,k,v,o,gate,up,down order) of a layer."""
    return 1000 + 7 * layer + j


def config1():
    """Single small layer: K = N = 256, M = 4.  W ~ N(0, 0.02) is drawn first,
    then X ~ N(0, 1), both from numpy's default_rng(0)."""
    rng = np.random.default_rng(0)
    W = (rng.standard_normal((256, 256)) * 0.02).astype(np.float32)
    X = rng.standard_normal((4, 256)).astype(np.float32)
    return W, X


def weights_np(N: int, K: int, sigma: float, seed: int) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return (rng.standard_normal((N, K), dtype=np.float32) * np.float32(sigma)).astype(np.float32)


def outlier_channels(K: int, seed: int, frac: float = 0.01) -> np.ndarray:
    """A seeded choice of round(frac*K) input channels (fixed across tokens)."""
    rng = np.random.default_rng(seed + 7919)
    n = int(round(frac * K))
    return np.sort(rng.choice(K, size=n, replace=False)).astype(np.int64)


def activations_np(M: int, K: int, seed: int, outlier_frac: float = 0.0,
                   outlier_scale: float = 20.0) -> np.ndarray:
    """X ~ N(0, 1); with outlier_frac > 0, that fraction of the K channels is
    multiplied by outlier_scale for every token."""
    rng = np.random.default_rng(seed)
    X = rng.standard_normal((M, K), dtype=np.float32)
    if outlier_frac > 0:
        ch = outlier_channels(K, seed, outlier_frac)
        X[:, ch] *= np.float32(outlier_scale)
    return X


def weights_torch(N: int, K: int, sigma: float, seed: int, device):
    """Same distribution as weights_np, drawn on the device by torch's
    generator (used where the fp32 matrices are too large to draw on the
    host: the full model stacks)."""
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    W = torch.randn((N, K), generator=g, device=device, dtype=torch.float32)
    W.mul_(sigma)
    return W


def activations_torch(M: int, K: int, seed: int, device, outlier_frac: float = 0.0,
                      outlier_scale: float = 20.0):
    import torch
    g = torch.Generator(device=device)
    g.manual_seed(seed)
    X = torch.randn((M, K), generator=g, device=device, dtype=torch.float32)
    if outlier_frac > 0:
        ch = torch.from_numpy(outlier_channels(K, seed, outlier_frac)).to(device)
        X[:, ch] *= outlier_scale
    return X


def random_ternary(N: int, K: int, seed: int, p_zero: float = 1.0 / 3.0) -> np.ndarray:
    rng = np.random.default_rng(seed)
    u = rng.random((N, K))
    T = np.where(u < p_zero, 0, np.where(u < (1 + p_zero) / 2, 1, -1))
    return T.astype(np.int8)


def random_int8(M: int, K: int, seed: int, lo: int = -127, hi: int = 127) -> np.ndarray:
    rng = np.random.default_rng(seed)
    return rng.integers(lo, hi + 1, size=(M, K), dtype=np.int64).astype(np.int8)
