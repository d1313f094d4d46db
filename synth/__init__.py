"""Seeded synthetic inputs for the SVDQuant W4A4 + low-rank linear and the W4A16 projection.

This module only draws random numbers and stores them in the 16-bit input format. It holds none
of the method's arithmetic (no smoothing, no decomposition, no quantization): the offline
decomposition and the layer itself live on each side that consumes these arrays, the oracle and
the product, independently.

Workloads. The pages measure end to end on trained diffusion transformers (FLUX.1-dev and
others); the layer shapes below stand in for those models with synthetic data of FLUX
proportions: 4096 image + 512 text tokens, hidden 3072, MLP 12288, a fused Q|K|V projection of
3 x 3072 outputs (concatenated Q then K then V along the output dimension, as the Diffusers blog
on Nunchaku describes for ``to_qkv``), and a 6 x 3072 adaptive-normalisation modulation
projection. Activations carry a few outlier channels, the phenomenon the SVDQuant overview figure
(stage 1) describes: a small number of input channels with much larger magnitude than the rest.

Recipe (all draws from ``numpy.random.Generator(PCG64(seed))`` in this fixed order):
  1. Z ~ N(0, 1), float64 [M, K]; the MLP down projection's input is GELU(Z) (exact erf form).
  2. Outlier channel set: ``n_outliers`` distinct channels drawn without replacement; those
     columns of X are multiplied by ``outlier_scale`` (after the GELU where there is one).
  3. W ~ N(0, 0.02), float64 [K, N] (second parameter of N is the standard deviation).
  4. bias ~ N(0, 0.01), float64 [N] (only where the configuration has a bias).
Every array is rounded to float32 and then to bfloat16 with round-to-nearest-even; bf16 arrays
are returned as their uint16 bit patterns.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Dict, Optional

import numpy as np

__all__ = ["LayerConfig", "CONFIGS", "make_layer_inputs", "bf16_bits_from_f32", "f32_from_bf16_bits",
           "random_bf16", "random_f32"]


@dataclasses.dataclass(frozen=True)
class LayerConfig:
    name: str
    M: int
    K: int
    N: int
    rank: int            # low-rank branch rank r (0 for the W4A16 projection)
    seed: int
    n_outliers: int = 0
    outlier_scale: float = 1.0
    gelu_input: bool = False
    has_bias: bool = True
    kind: str = "w4a4"   # "w4a4" (SVDQuant linear) or "w4a16" (AWQ-style projection)

    def with_rank(self, r: int) -> "LayerConfig":
        return dataclasses.replace(self, rank=r, name=f"{self.name.split('_r')[0]}_r{r}")


def _outliers(K: int) -> int:
    return int(round(0.01 * K))


CONFIGS: Dict[str, LayerConfig] = {
    # tiny SVDQuant linear: 4 outlier channels x20, rank 16
    "tiny": LayerConfig("tiny", 256, 256, 512, 16, seed=0, n_outliers=4, outlier_scale=20.0),
    # attention output projection, 4096 image + 512 text tokens
    "attn": LayerConfig("attn", 4608, 3072, 3072, 32, seed=1, n_outliers=_outliers(3072), outlier_scale=30.0),
    # MLP up projection
    "up": LayerConfig("up", 4608, 3072, 12288, 32, seed=2, n_outliers=_outliers(3072), outlier_scale=30.0),
    # MLP down projection, input = GELU of N(0,1)
    "down": LayerConfig("down", 4608, 12288, 3072, 32, seed=3, n_outliers=_outliers(12288), outlier_scale=30.0,
                        gelu_input=True),
    # fused Q|K|V projection; rank swept over 32 / 128 / 256 on one problem
    "qkv_r32": LayerConfig("qkv_r32", 4608, 3072, 9216, 32, seed=4, n_outliers=_outliers(3072), outlier_scale=30.0),
    "qkv_r128": LayerConfig("qkv_r128", 4608, 3072, 9216, 128, seed=4, n_outliers=_outliers(3072), outlier_scale=30.0),
    "qkv_r256": LayerConfig("qkv_r256", 4608, 3072, 9216, 256, seed=4, n_outliers=_outliers(3072), outlier_scale=30.0),
    # adaLN modulation projection, weight-only 4-bit, no low-rank branch, no bias
    "awq": LayerConfig("awq", 16, 3072, 18432, 0, seed=5, has_bias=False, kind="w4a16"),
}


def bf16_bits_from_f32(a: np.ndarray) -> np.ndarray:
    """Round float32 values to bfloat16 (nearest, ties to even); returns uint16 bit patterns."""
    u = np.ascontiguousarray(a, dtype=np.float32).view(np.uint32).astype(np.uint64)
    u = u + 0x7FFF + ((u >> 16) & 1)
    return (u >> 16).astype(np.uint16)


def f32_from_bf16_bits(b: np.ndarray) -> np.ndarray:
    """Widen bfloat16 bit patterns to float32 values (exact)."""
    return (np.ascontiguousarray(b, dtype=np.uint16).astype(np.uint32) << 16).view(np.float32)


def _gelu_erf(z: np.ndarray) -> np.ndarray:
    from scipy.special import erf
    return 0.5 * z * (1.0 + erf(z / math.sqrt(2.0)))


def make_layer_inputs(cfg: LayerConfig, seed: Optional[int] = None, M: Optional[int] = None) -> Dict[str, np.ndarray]:
    """Draw one layer's raw inputs.

    Returns ``x`` (uint16 bf16 bits [M, K]), ``w`` (uint16 bf16 bits [K, N]), ``bias`` (uint16 bf16 bits
    [N] or None) and ``outliers`` (int64 channel indices). ``M`` overrides the token count (the
    same channel statistics, fewer or more rows) and ``seed`` the configuration's seed.
    """
    rng = np.random.Generator(np.random.PCG64(cfg.seed if seed is None else seed))
    m = cfg.M if M is None else M
    z = rng.standard_normal((m, cfg.K))
    x = _gelu_erf(z) if cfg.gelu_input else z
    outl = np.sort(rng.choice(cfg.K, size=cfg.n_outliers, replace=False)) if cfg.n_outliers else np.zeros(0, np.int64)
    if cfg.n_outliers:
        x[:, outl] *= cfg.outlier_scale
    w = rng.normal(0.0, 0.02, size=(cfg.K, cfg.N))
    bias = rng.normal(0.0, 0.01, size=cfg.N) if cfg.has_bias else None
    return {
        "x": bf16_bits_from_f32(x.astype(np.float32)),
        "w": bf16_bits_from_f32(w.astype(np.float32)),
        "bias": None if bias is None else bf16_bits_from_f32(bias.astype(np.float32)),
        "outliers": outl.astype(np.int64),
    }


def random_bf16(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    """N(0, scale) values rounded to bf16; uint16 bits."""
    rng = np.random.Generator(np.random.PCG64(seed))
    return bf16_bits_from_f32((rng.standard_normal(shape) * scale).astype(np.float32))


def random_f32(shape, seed: int, scale: float = 1.0) -> np.ndarray:
    rng = np.random.Generator(np.random.PCG64(seed))
    return (rng.standard_normal(shape) * scale).astype(np.float32)
