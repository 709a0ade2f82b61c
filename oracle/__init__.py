"""Plain float64 CPU oracle for the HySparse2 inner-level attention path.

Test infrastructure only: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py, never by the library.  See hs2_oracle.py.
"""
from .hs2_oracle import *  # noqa: F401,F403
from .hs2_oracle import __all__  # noqa: F401
