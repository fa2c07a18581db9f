"""Float64 CPU oracle of the POET-X linear layer (test infrastructure only).

Only tests, the smoke check and the benchmark's CPU-baseline leg may import
this package. The GPU product path never imports, calls or links it.
"""
from .poetx_oracle import *  # noqa: F401,F403
