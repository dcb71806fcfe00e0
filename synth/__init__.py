"""Seeded synthetic inputs for the HARD-KV decode step.

This package holds the workload definitions and the input generator that both
the CPU oracle (under ``oracle/``) and the HIP library are fed from.  It holds
none of the method's arithmetic: it only draws Gaussian caches and queries,
plants heavy tokens, and records the sizes and knobs of each workload.
"""

from .configs import WORKLOADS, Workload, get_workload  # noqa: F401
from .generate import Inputs, make_inputs, tiny_workload  # noqa: F401
