"""CPU oracle of the USAF sparse MoE step (test infrastructure only).

Only tests/, __graft_entry__.smoke() and bench.py's CPU-baseline leg may import
this package.  It never imports the HIP path.
"""
from .usaf_oracle import *  # noqa: F401,F403
from . import usaf_oracle  # noqa: F401
