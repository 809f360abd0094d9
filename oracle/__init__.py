"""fp64 CPU oracle for the batched token sampler.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the product path.
"""
from . import commit, sampler  # noqa: F401
