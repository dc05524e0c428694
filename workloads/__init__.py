"""Seeded synthetic workloads shared by the tests, smoke() and bench.py.

This package only draws inputs.  It holds none of the method's arithmetic
(no pooling, scoring, selection or attention); the oracle and the HIP library
each compute everything from the tensors drawn here.
"""
from .configs import WORKLOADS, Workload  # noqa: F401
from .synth import (  # noqa: F401
    decode_inputs,
    drift_walk,
    prefill_inputs,
    random_decode_case,
    random_prefill_case,
)
