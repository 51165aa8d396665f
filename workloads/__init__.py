"""Seeded synthetic input generators shared by the tests, the benchmark and
the oracle's callers.  Holds no arithmetic of the method itself."""
from .synth import (  # noqa: F401
    Config, CONFIGS, config, small_config, normal_at, channel_sigma,
    dense_rotations, channel_orders, kv_tokens, queries, head_major,
)
