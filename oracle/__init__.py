"""CPU float64 oracle for the routed Mixture-of-Experts FFN forward.

TEST INFRASTRUCTURE ONLY. Only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import this package. The GPU library never calls it, and it
shares no code with the GPU library.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
