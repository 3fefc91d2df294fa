"""fp64 CPU oracle for exact attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg import
this package.  It imports nothing from the HIP library.
"""
from .attention_ref import *  # noqa: F401,F403
from .attention_ref import __all__  # noqa: F401
