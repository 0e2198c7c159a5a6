"""Float64 CPU oracle for the PowerSGD step, the per-resblock gradient scaling at block
boundaries and the optimizer step that consumes the decompressed gradient. TEST
INFRASTRUCTURE ONLY.

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import this package.
The HIP library never calls it, and the two share no code. The product path fails loudly when
the HIP library is missing; it never falls back to this oracle.
"""
from . import adam, blockscale, powersgd  # noqa: F401
from .adam import *  # noqa: F401,F403
from .blockscale import *  # noqa: F401,F403
from .powersgd import *  # noqa: F401,F403

__all__ = list(powersgd.__all__) + list(blockscale.__all__) + list(adam.__all__)
