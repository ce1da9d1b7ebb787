"""MI355X (gfx950) routed Mixture-of-Experts layer forward.

The compute path is libmoe.so (hand-written HIP kernels behind a C ABI, see
include/moe.h); `binding` marshals torch device tensors into it and
`workloads` draws the seeded synthetic inputs.
"""
from . import binding, workloads  # noqa: F401
from .binding import (moe_combine, moe_grouped_ffn, moe_layer_forward, moe_permute,  # noqa: F401
                      moe_route, LayerForward, MoEError)
