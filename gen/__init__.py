"""Seeded synthetic inputs shared by the oracle's tests, the GPU parity tests and the bench.

This package draws random numbers and names workload sizes; it contains no part of the
balanced expert-parallel method itself.
"""

from .configs import Workload, WORKLOADS, BY_NAME, TINY, SMALL, DSV3, KIMI, DECODE  # noqa: F401
from .routing import make_routing, make_balanced_routing, realised_maxvio  # noqa: F401
from .tensors import (make_hidden, make_scales, make_grads, bf16_bits,  # noqa: F401
                      bits_to_bf16)
