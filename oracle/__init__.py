"""Float64 CPU oracle for the PowerSGD step. TEST INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The HIP library never calls it, and the two share no code. The product path fails loudly when
the HIP library is missing; it never falls back to this oracle.
"""
from .powersgd import *  # noqa: F401,F403
from .powersgd import __all__  # noqa: F401
