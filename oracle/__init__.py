"""fp64 CPU oracle for the attention path (test infrastructure only).

Only the tests, the smoke check and the benchmark's CPU-baseline leg may use
this package; the product path never imports it.
"""
from .attn64 import *  # noqa: F401,F403
