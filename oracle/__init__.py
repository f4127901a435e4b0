"""CPU oracle (test infrastructure only; see moe_oracle.py for what it computes and why).

Only the test-suite, the entry point's smoke check and the benchmark's CPU-baseline leg
may import this package.  The product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import CombineState, combine_release, combine_token  # noqa: F401
