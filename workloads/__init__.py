"""Seeded synthetic workloads for the sharded optimizer step.

This package only describes inputs: parameter-tensor shape lists, run settings
and seeded generators for parameters, gradients and injected non-finite values.
It holds none of the optimizer step's arithmetic, so both the GPU path and the
CPU oracle can draw their inputs from it without sharing any of the method.
"""

from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from .gen import make_grads, make_params  # noqa: F401
