"""Seeded synthetic inputs and workload shapes for the Gemma 4 attention layer.

This module holds no arithmetic of the attention method: only the workload
shapes (taken from the model variants the pages describe) and seeded random
draws.  Both the HIP library's tests/bench and the fp64 oracle consume what
it produces; neither side's code lives here.
"""

from .configs import WORKLOADS, Workload, get  # noqa: F401
from .gen import (normal_bf16, norm_weight, decode_lengths,  # noqa: F401
                  seed_key, to_f64)
