"""Seeded synthetic inputs for the MoE dispatch -> expert -> combine path.

This module is the only code that both the oracle side (tests, CPU baseline)
and the GPU side use.  It holds no step of the path itself: it only draws
activations, routing decisions and expert weights.  Routing (top-k over
router scores) happens upstream of dispatch, so it is input synthesis here.

Draw order per config: x, then routing, then weights.  x and routing come
from ``numpy.random.default_rng(seed)``; weights from per-expert
``torch.Generator`` streams seeded from (seed, expert) on the device that
will hold them, so full-size weights are drawn on the GPU in milliseconds
and copied to the host only where the oracle needs them.  All bf16 values
are fp32 draws rounded to nearest even by torch's conversion.
"""
from .configs import CONFIGS, MoEConfig, get_config  # noqa: F401
from .gen import (  # noqa: F401
    activations,
    bf16_bits,
    expert_weights,
    forced_edge_routing,
    routing,
)
