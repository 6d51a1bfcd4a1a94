"""CPU oracle for the NVFP4 W4A4 linear layer (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may import
this package; the product path (the HIP library and its binding) never does.
"""
from .nvfp4 import *  # noqa: F401,F403
from . import nvfp4  # noqa: F401
