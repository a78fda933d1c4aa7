"""Float64 CPU oracle for absorbed-MLA decode (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the product path never does.
"""
from .mla_oracle import *  # noqa: F401,F403
from . import mla_oracle  # noqa: F401
