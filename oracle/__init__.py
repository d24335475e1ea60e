"""fp64 CPU oracle for LSH-sampled decode attention.

Test infrastructure only: imported by ``tests/``, ``__graft_entry__.smoke()``
and the ``cpu_baseline`` leg of ``bench.py``, never by the library.
"""
from .lsh_oracle import *  # noqa: F401,F403
from . import lsh_oracle  # noqa: F401
