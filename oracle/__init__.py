"""Float64 CPU oracle for LRKV compressed-cache attention.

TEST INFRASTRUCTURE ONLY: imported by ``tests/``, ``__graft_entry__.smoke()``
and the CPU-baseline leg of ``bench.py``, never by the product package.
"""
from .lrkv_oracle import *  # noqa: F401,F403
from .lrkv_oracle import __all__  # noqa: F401
