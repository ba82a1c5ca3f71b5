"""Seeded synthetic inputs for paged decode attention.

This package holds only input construction: decode-step configurations, sequence
lengths, block tables, slot ids of the new tokens and the random K/V/Q values.
It contains none of the attention arithmetic, so both the CPU oracle side and the
HIP side of the tests can draw their inputs from it without sharing any method code.
"""

from .configs import CONFIGS, DecodeConfig, config_by_name  # noqa: F401
from .gen import (  # noqa: F401
    DecodeCase,
    make_case,
    nan_bits,
    round_to_bits,
    bits_dtype_name,
    fork_shape,
    is_fork,
)
