"""fp64 CPU oracle of the MoE FFN layer.

TEST INFRASTRUCTURE: only the test suite, the smoke check of the package
entry module and the CPU-baseline leg of the benchmark may import it.  The
product path never does.
"""
from .moe_oracle import *  # noqa: F401,F403
from .moe_oracle import __all__  # noqa: F401
