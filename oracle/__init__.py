"""fp64 CPU oracle for the fused LM-head GRPO / GSPO head loss.

TEST INFRASTRUCTURE: only tests/, __graft_entry__.smoke() and bench.py's
cpu_baseline leg may import it.  It shares no code with the GPU library.
Every function is pinned by the CPU tests in tests/test_oracle_*.py.
"""
from .grpo_oracle import *  # noqa: F401,F403
from .grpo_oracle import __all__  # noqa: F401
