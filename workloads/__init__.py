"""Seeded synthetic inputs for EntmaxKV paged decode.

This package only draws random numbers and lays them out as a paged KV pool
(pool of physical page slots, per-sequence page tables, sequence lengths and
queries).  It holds none of the method's arithmetic: no scores, bounds,
metadata, selection or attention.  Both the fp64 oracle tests and the HIP
path's tests and benchmark take their inputs from here.
"""
from .synth import (  # noqa: F401
    WORKLOADS,
    Workload,
    PagedInputs,
    workload,
    generate,
    append_token,
    draw_fresh_queries,
)
