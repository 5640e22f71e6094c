"""CPU oracle for the HSA denoise-iteration path (test infrastructure only).

Only tests, ``__graft_entry__.smoke()`` and ``bench.py``'s cpu_baseline leg use it.
"""
from .hsa_oracle import *  # noqa: F401,F403
