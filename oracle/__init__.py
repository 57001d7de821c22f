"""CPU oracle (float64) for the S4R compressed-KV path.

TEST INFRASTRUCTURE ONLY: used by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  The product path never imports it."""
from .s4r import *  # noqa: F401,F403
from .s4r import Cache, rnd  # noqa: F401
