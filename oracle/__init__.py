"""CPU oracle for the sparse MoE FFN layer — test infrastructure only.

Only ``tests/``, ``__graft_entry__.smoke()`` and the CPU-baseline leg of
``bench.py`` may import this package.  It shares no code with the HIP path.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import TIE_GAP  # noqa: F401
