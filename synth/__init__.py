"""Seeded synthetic inputs shared by the oracle, the tests and the benchmark.

This package holds data only: model shapes, pair configurations, seeded
random-init weights and seeded prompts.  It contains none of the method's
arithmetic (no normalisation, attention, sampling or acceptance), so both the
CPU oracle and the HIP path can consume its outputs without sharing code.
"""
from .configs import ModelShape, PairConfig, CONFIGS, get_config, tiny_shape
from .weights import make_weights, WEIGHT_KEYS
from .prompts import make_prompts

__all__ = ["ModelShape", "PairConfig", "CONFIGS", "get_config", "tiny_shape",
           "make_weights", "WEIGHT_KEYS", "make_prompts"]
