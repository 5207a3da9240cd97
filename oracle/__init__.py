"""CPU oracle for the ISPA hot path: test infrastructure only.

Plain fp64 numpy code that restates what the pages define.  It is
imported by ``tests/``, by ``__graft_entry__.smoke()`` and by the
``cpu_baseline`` leg of ``bench.py``, and by nothing else; the HIP library
never calls it and it never calls the HIP library.
"""
from .ispa_oracle import *  # noqa: F401,F403
