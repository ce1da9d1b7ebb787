"""CPU oracles (float64, numpy): the routed-MoE layer forward, the expert-FFN
backward, the whole layer backward, and Muon's Newton-Schulz orthogonalisation
of whole matrices.

Test infrastructure: only the tests, the smoke check and the benchmark's
CPU-baseline leg may import it.  The product path never does.
"""
from . import moe_backward_oracle, moe_layer_backward_oracle, moe_oracle, muon_oracle  # noqa: F401
