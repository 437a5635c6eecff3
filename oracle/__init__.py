"""fp64 oracle of the LM-head log-prob / entropy head.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and ``bench.py``'s ``cpu_baseline`` leg, never by the product path
(``cross_entropy_amd``), and it imports nothing from it.
"""
from . import lmhead_oracle, bruteforce  # noqa: F401
from .lmhead_oracle import (  # noqa: F401
    backward,
    chunk_ranges,
    forward,
    forward_backward,
    loss,
    valid_targets,
    widen_bf16,
)
