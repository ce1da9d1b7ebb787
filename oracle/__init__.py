"""CPU oracle of the routed-MoE layer forward (float64, numpy).

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  The product path never does.
"""
from . import moe_oracle  # noqa: F401
