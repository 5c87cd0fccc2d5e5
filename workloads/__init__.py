"""Seeded synthetic workloads for the HiSparse sparse-decode path.

This package only draws random structure and random values: request lengths,
block tables (page permutations), top-k position lists, which positions start
out in each request's hot buffer, query/KV/logit tensors.  It holds none of the
method's arithmetic (no block-table address mapping, no hit/miss test, no LRU,
no attention, no argmax).  Both the CPU oracle's tests and the GPU harness take
their inputs from here; each side derives everything else with its own code.
"""

from .synth import (  # noqa: F401
    CONFIGS,
    Workload,
    WorkloadSpec,
    generate,
    spec,
)
