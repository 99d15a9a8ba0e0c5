"""Seeded synthetic inputs shared by the tests, the bench and the smoke check.

This package only draws random numbers and converts their storage type.  It
holds none of the decode path's arithmetic (no bit assignment, no packing, no
dequantisation, no product): both the HIP library and the CPU oracle receive
the arrays it produces, and neither imports the other.
"""

from .workloads import *  # noqa: F401,F403
