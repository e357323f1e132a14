"""Seeded synthetic inputs for the shared-KV cross-attention path.

This package holds no arithmetic of the method: it only draws random numbers
(NumPy PCG64 streams spawned from one seed), rounds them to the storage dtype and
lays them out in the shared-cache pool format. Both the fp64 oracle and the HIP
path consume what it returns.
"""
from .workloads import WORKLOADS, Workload, ragged_lengths  # noqa: F401
from .inputs import (  # noqa: F401
    PrefillCase,
    DecodeCase,
    make_prefill_case,
    make_chunk_case,
    make_decode_case,
    to_f64,
    to_f32,
)
