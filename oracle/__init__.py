"""fp64 CPU oracle for causal linear attention (test infrastructure only).

Only ``tests/``, ``__graft_entry__.smoke()`` and ``bench.py``'s
``cpu_baseline`` leg may import this package; the HIP library never does.
"""

from .linattn_oracle import *  # noqa: F401,F403
from .linattn_oracle import __all__  # noqa: F401
