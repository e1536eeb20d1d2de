"""CPU fp64 oracle of the VDN hybrid attention forward.

TEST INFRASTRUCTURE: imported only by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The product path never imports it.
"""
from .vdn_oracle import *  # noqa: F401,F403
