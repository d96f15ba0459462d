"""fp64 CPU oracle for fixed-m attention forward.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()`` and the
``cpu_baseline`` leg of ``bench.py``.  The HIP product path never imports, calls or links it.
"""
from .fixedm_oracle import *  # noqa: F401,F403
