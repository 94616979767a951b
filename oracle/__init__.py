"""CPU oracle of the sparse-linear hybrid attention forward and of its gradients.

TEST INFRASTRUCTURE ONLY: imported by tests/, __graft_entry__.smoke() and the
cpu_baseline leg of bench.py.  Nothing in the product path imports it.
"""
from .sla_oracle import *  # noqa: F401,F403
from . import sla_oracle  # noqa: F401
from . import sla_backward  # noqa: F401
