"""Seeded synthetic workloads for MoE token dispatch/combine.

This package only draws inputs (token rows, top-k expert ids, gate weights)
and names the workload shapes. It holds none of the dispatch/combine
arithmetic, so both the CPU oracle and the GPU path can take their inputs
from it without sharing any of the method's code.
"""

from .workloads import WORKLOADS, Workload, make_fp8_payload, make_inputs  # noqa: F401
