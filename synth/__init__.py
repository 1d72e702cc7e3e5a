"""Seeded synthetic workloads shared by the tests, the bench and the CPU oracle.

This package draws random numbers and shapes them into the input
distributions of the five workloads (query/key/value vectors, write strengths,
retention gates, slot permutations).  It holds none of the method's
arithmetic: no recurrence, no quantizer, no calibration statistic.
"""
from .inputs import (  # noqa: F401
    WORKLOADS,
    Workload,
    workload,
    step_inputs,
    warmup_inputs,
    calib_inputs,
    slot_ids,
    gate_params,
)
