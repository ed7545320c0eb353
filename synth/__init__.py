"""Seeded synthetic layers (weights + calibration activations) for the AWQ scale search.

This package holds random draws only: no quantisation, statistics, scaling or loss
arithmetic lives here.  Both the CPU oracle's tests and the GPU path's tests and
benchmark take their inputs from it, so the two sides always see the same fp16 arrays.
"""
from .awq_configs import (CONFIGS, LayerSpec, Layer, make_layer, config_layers, row_subset,
                          small_spec, alpha_grid)

__all__ = ["CONFIGS", "LayerSpec", "Layer", "make_layer", "config_layers", "row_subset",
           "small_spec", "alpha_grid"]
