"""Seeded synthetic inputs for the routed MoE layer forward.

This package is shared by the tests, the benchmark and the smoke check.  It only
draws random numbers and lays them out in the library's input layout; it holds
none of the layer's arithmetic, and it imports neither the GPU library nor the
CPU oracle.
"""
from .configs import (CONFIGS, MLP_CONFIGS, ExpertMlpConfig, LayerConfig, PoolConfig,  # noqa: F401
                      by_name)
from .gen import (expert_mlp_routing, gen_expert_mlp, gen_layer, gen_pool, layer_shapes,  # noqa: F401
                  small_int_tensor)
