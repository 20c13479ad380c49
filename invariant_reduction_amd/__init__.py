"""invariant_reduction_amd: deterministic, batch-invariant and
tensor-parallel-invariant reductions for MI355X (gfx950).

The compute runs in ``libdetred.so`` (hand-written HIP kernels behind the C
ABI declared in ``include/detred.h``); ``invariant_reduction_amd.detred`` is
a thin ctypes binding that passes torch device pointers and streams to it.
``inputs`` holds the seeded synthetic input generators.
"""
from . import inputs  # noqa: F401
