"""Seeded synthetic stand-ins for the calibration data of one linear layer.

The pages calibrate on real text (WikiText-2 samples for AutoAWQ, a few hundred to a
thousand 2048-token texts in another walkthrough); neither the data nor the model weights
exist here.  Each workload below is a synthetic layer with the shape, weight spread and
activation outlier structure of the five named cases:

  W   fp16 [out_features][in_features]      row-major, in_features contiguous
  X   fp16 [n_tokens][in_features]          row-major (the pages' X^T), in_features contiguous

Recipe (all draws in float64, then scaled, cast to float32, then to float16 with
round-to-nearest-even, which is what numpy's astype does):

  rng_j = numpy.random.default_rng(1000*c + 10*layer + j)
     j = 1 weights, 2 activations, 3 outlier channel choice and factors, 4 row subset
  W  = sigma_w * N(0, 1)
  X  = N(0, 1)  or Student-t(nu=4); drawn in blocks of ROW_BLOCK rows so that the stream
       does not depend on available memory
  outliers: n_out = round(frac * in_features) channels chosen without replacement; the
       whole column (all tokens) is multiplied by its factor before the casts.

Nothing here computes anything the quantiser, the statistics or the loss compute.
"""
from __future__ import annotations

import dataclasses
import math
from typing import Optional

import numpy as np

ROW_BLOCK = 1024  # rows per draw call; part of the recipe (fixes the random stream)


@dataclasses.dataclass(frozen=True)
class LayerSpec:
    """One synthetic linear layer and its quantisation settings."""

    name: str
    out_features: int          # M
    in_features: int           # K
    n_tokens: int              # N
    w_sigma: float
    x_dist: str                # "normal" or "t4"
    outlier_count: int         # channels whose activations are amplified
    outlier_factor: object     # float, or ("loguniform", lo, hi)
    w_bit: int
    group_size: int
    zero_point: int
    seed_base: int             # 1000*c + 10*layer
    n_alpha: int = 20


@dataclasses.dataclass
class Layer:
    spec: LayerSpec
    W: np.ndarray              # float16 [M][K]
    X: np.ndarray              # float16 [N][K]
    outlier_channels: np.ndarray
    outlier_factors: np.ndarray


def _spec(name, c, layer, M, K, N, w_sigma, x_dist, frac_or_count, factor, w_bit, g, zp):
    if isinstance(frac_or_count, float):
        n_out = int(round(frac_or_count * K))
    else:
        n_out = int(frac_or_count)
    return LayerSpec(name, M, K, N, w_sigma, x_dist, n_out, factor, w_bit, g, zp,
                     1000 * c + 10 * layer)


# The five workloads; the headline case is "c2", a 4096 x 4096 layer with 4096 tokens.
CONFIGS = {
    "c1": [_spec("c1", 1, 0, 512, 512, 256, 0.02, "normal", 5, 20.0, 4, 128, 0)],
    "c2": [_spec("c2", 2, 0, 4096, 4096, 4096, 0.02, "normal", 0.01,
                 ("loguniform", 10.0, 50.0), 4, 128, 1)],
    "c3": [_spec("c3_up", 3, 0, 11008, 4096, 16384, 0.02, "t4", 0.01, 20.0, 4, 128, 1),
           _spec("c3_down", 3, 1, 4096, 11008, 16384, 0.02, "t4", 0.01, 20.0, 4, 128, 1)],
    "c4": [_spec("c4", 4, 0, 28672, 8192, 65536, 0.015, "normal", 0.005, 30.0, 4, 128, 1)],
    "c5": [_spec("c5", 5, 0, 13824, 5120, 32768, 0.02, "normal", 0.01, 20.0, 3, 64, 1)],
}


def _draw_rows(rng: np.random.Generator, n_rows: int, n_cols: int, dist: str,
               scale: float, col_factors: Optional[np.ndarray]) -> np.ndarray:
    out = np.empty((n_rows, n_cols), dtype=np.float16)
    for r0 in range(0, n_rows, ROW_BLOCK):
        r1 = min(n_rows, r0 + ROW_BLOCK)
        if dist == "normal":
            blk = rng.standard_normal((r1 - r0, n_cols))
        elif dist == "t4":
            blk = rng.standard_t(4.0, (r1 - r0, n_cols))
        else:
            raise ValueError(dist)
        if scale != 1.0:
            blk *= scale
        if col_factors is not None:
            blk *= col_factors[None, :]
        out[r0:r1] = blk.astype(np.float32).astype(np.float16)
    return out


def make_layer(spec: LayerSpec) -> Layer:
    """Generate one layer deterministically from its spec."""
    M, K, N = spec.out_features, spec.in_features, spec.n_tokens
    rng_w = np.random.default_rng(spec.seed_base + 1)
    rng_x = np.random.default_rng(spec.seed_base + 2)
    rng_o = np.random.default_rng(spec.seed_base + 3)

    n_out = min(spec.outlier_count, K)
    chans = rng_o.choice(K, n_out, replace=False) if n_out > 0 else np.zeros(0, np.int64)
    if isinstance(spec.outlier_factor, tuple):
        kind, lo, hi = spec.outlier_factor
        assert kind == "loguniform"
        facs = np.exp(rng_o.uniform(math.log(lo), math.log(hi), n_out))
    else:
        facs = np.full(n_out, float(spec.outlier_factor))
    col = np.ones(K, dtype=np.float64)
    col[chans] = facs

    W = _draw_rows(rng_w, M, K, "normal", spec.w_sigma, None)
    X = _draw_rows(rng_x, N, K, spec.x_dist, 1.0, col if n_out > 0 else None)
    return Layer(spec, W, X, np.asarray(chans), np.asarray(facs))


def config_layers(name: str):
    """All layers of a named workload ("c1" ... "c5")."""
    return [make_layer(s) for s in CONFIGS[name]]


def row_subset(spec: LayerSpec, n_rows: int = 512) -> np.ndarray:
    """Seeded sorted subset of output rows (used where the full layer is too big for the
    CPU oracle; the loss is a sum over rows, so a row subset is checked exactly)."""
    rng = np.random.default_rng(spec.seed_base + 4)
    n_rows = min(n_rows, spec.out_features)
    return np.sort(rng.choice(spec.out_features, n_rows, replace=False))


def small_spec(name: str, M: int, K: int, N: int, w_bit: int = 4, group_size: int = 128,
               zero_point: int = 1, seed: int = 7, x_dist: str = "normal",
               outlier_count: int = 3, outlier_factor=20.0, w_sigma: float = 0.02,
               n_alpha: int = 20) -> LayerSpec:
    """A layer of arbitrary (small) shape drawn with the same recipe, for parity cases."""
    return LayerSpec(name, M, K, N, w_sigma, x_dist, outlier_count, outlier_factor,
                     w_bit, group_size, zero_point, 100000 + 10 * seed, n_alpha)


def alpha_grid(n: int = 20) -> np.ndarray:
    """Evenly spaced grid over [0, 1] with both ends, as float32."""
    if n == 1:
        return np.zeros(1, dtype=np.float32)
    return (np.arange(n, dtype=np.float64) / (n - 1)).astype(np.float32)
