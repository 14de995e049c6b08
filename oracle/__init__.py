"""CPU oracle for the paged DSA step -- test infrastructure only.

Only the tests, the smoke check and the benchmark's CPU-baseline leg import
this package; the product path never does.
"""
from . import dsa_oracle  # noqa: F401
