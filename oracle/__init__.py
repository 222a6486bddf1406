"""fp64 CPU oracle for the InfLLM-V2 sparse-attention path.

TEST INFRASTRUCTURE ONLY.  Nothing in the product path may import, call, link
or execute this package; only the tests, the smoke check and the benchmark's
CPU-baseline leg do.  It shares no code with the HIP library or its binding.
"""
from .reference import *  # noqa: F401,F403
