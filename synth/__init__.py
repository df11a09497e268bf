"""Seeded synthetic inputs shared by the GPU path's tests/bench and by the oracle.

This package only draws random numbers, rounds them to the storage formats with torch's own
casts and lays them out in 64-token pages.  It holds no part of the method's arithmetic.
"""
from .workloads import (PAGE, TINY, DECODE32K, PREFILL64K, DECODE1M, RAGGED, NAMES, Shape,
                        Workload, workload, reduced, seed_of, ragged_lengths)
from .gen import Inputs, make

__all__ = ["PAGE", "TINY", "DECODE32K", "PREFILL64K", "DECODE1M", "RAGGED", "NAMES", "Shape",
           "Workload", "workload", "reduced", "seed_of", "ragged_lengths", "Inputs", "make"]
