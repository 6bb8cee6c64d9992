"""CPU oracle (test infrastructure only) for the W4A16 group-128 path.

Only ``tests/``, ``__graft_entry__.smoke()`` and the benchmark's CPU-baseline
leg import this package.  It shares no code with the HIP library.
"""
from .w4a16_oracle import *  # noqa: F401,F403
from .w4a16_oracle import GROUP  # noqa: F401
