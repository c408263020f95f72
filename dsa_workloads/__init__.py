"""Seeded synthetic workloads shared by the tests, the bench and the smoke check.

Holds shapes and random-input recipes only; no arithmetic of the method.
"""
from .configs import CONFIGS, BY_NAME, DSAConfig, scaled  # noqa: F401
from .generate import (  # noqa: F401
    generate, generate_projection_inputs, random_score_rows, quantize_e4m3_rows, plant_positions,
)
