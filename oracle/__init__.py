"""CPU oracle for MC-Sparse — test infrastructure only.

Only tests/, __graft_entry__.smoke() and the CPU-baseline leg of bench.py may
import this package.  The GPU library never uses it.
"""

from .mcs_oracle import *  # noqa: F401,F403
from .mcs_oracle import HASH_BITS, GroupSelection, HeadMeta  # noqa: F401
