"""Float64 CPU oracle for the DSA layer.

TEST INFRASTRUCTURE: imported only by ``tests/``, ``__graft_entry__.smoke()`` and the
CPU-baseline leg of ``bench.py``.  The library itself never imports it.
"""
from .dsa_oracle import *  # noqa: F401,F403
