"""CPU oracle for the fused W4A16 MoE layer -- test infrastructure only.

Plain, slow, float64 NumPy (plus a pure-Python brute force for tiny shapes)
written from the definitions on the pages.  Only tests/, the smoke check
and the benchmark's CPU-baseline leg may import it; the library and its
Python binding never do, and share no code, table or helper with it.
"""
from . import formats, moe, brute  # noqa: F401
