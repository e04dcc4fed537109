"""CPU oracle for grouped-query fused attention (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import this package; the product path never does.
"""
from .gqa_ref import *  # noqa: F401,F403
from .gqa_ref import __all__  # noqa: F401
