"""Seeded synthetic inputs shared by the HIP path's tests/bench and the oracle.

Holds input generation only (no FFN arithmetic)."""
from .configs import CONFIGS, ORDER, NOISE_VAR, StackConfig, scaled  # noqa: F401
from .gen import (Layer, make_layer, make_tokens, make_decision_values, quantize_q4_0,  # noqa: F401
                  powerlaw_profile, expected_top_share, chain_activation, solve_alpha, layer_mean,
                  seed_of)
