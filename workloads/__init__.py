"""Seeded synthetic inputs shared by the tests, the benchmark and the oracle
checks.  This package only draws random structure and tensors and lays them
out as a caller would hand them over (paged caches, page tables, mask
buffers); it holds none of the attention or mask-compilation arithmetic and
imports neither the oracle nor the library.
"""

from .gen import *  # noqa: F401,F403
