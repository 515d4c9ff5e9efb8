"""fp64 CPU oracle for dynamic bifocal RoPE attention.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg use it. It shares no code with the HIP library.
"""
from .bifocal_oracle import *  # noqa: F401,F403
from .bifocal_oracle import __all__  # noqa: F401
