"""Seeded synthetic inputs for the routed MoE layer forward.

This package is shared by the tests, the benchmark and the smoke check.  It only
draws random numbers and lays them out in the library's input layout; it holds
none of the layer's arithmetic, and it imports neither the GPU library nor the
CPU oracle.
"""
from .configs import CONFIGS, LayerConfig, PoolConfig, by_name  # noqa: F401
from .gen import gen_layer, gen_pool, layer_shapes  # noqa: F401
