"""fp64 CPU oracle of the sparse MoE FFN layer forward.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's cpu_baseline leg may
import it. It imports nothing from the GPU library, and the GPU library never imports it.
"""
from .moe_ref import *  # noqa: F401,F403
from . import moe_ref  # noqa: F401
