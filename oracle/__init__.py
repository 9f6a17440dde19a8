"""CPU oracle for the LoPA branch-verification step (test infrastructure).

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's
CPU-baseline leg may import this package.  The GPU library never does.
"""
from .lopa_oracle import *  # noqa: F401,F403
from .lopa_oracle import MASK  # noqa: F401
