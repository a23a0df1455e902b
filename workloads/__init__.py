"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

Holds shapes and random draws only; no step of the method is computed here.
"""
from .configs import CONFIGS, FocusConfig, get, scaled  # noqa: F401
from .gen import (Inputs, Metadata, draw_masked, draw_metadata,  # noqa: F401
                  draw_yield,
                  make_inputs,
                  make_layer, seed_for, to_f32_numpy, torch_dtype)
