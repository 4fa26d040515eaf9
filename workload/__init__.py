"""Seeded synthetic inputs for the MXFP4 latent-MoE layer (shared by tests, bench and smoke)."""
from .gen import SHAPES, LayerShape, make_inputs, sample_tokens, tie_tokens  # noqa: F401
