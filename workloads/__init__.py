"""Seeded synthetic inputs for the KDA forward (shared by tests and bench).

This package only draws random numbers and lays them out.  It holds none of
the method's arithmetic, so both the oracle side and the HIP side may be fed
from it without sharing any computation.
"""
from .kda_inputs import CONFIGS, KDAInputs, make_inputs, make_config, round_bf16  # noqa: F401
