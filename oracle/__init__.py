"""CPU oracle of the routed MoE layer forward -- TEST INFRASTRUCTURE ONLY.

Only the tests, the smoke check and the benchmark's CPU-baseline leg may import
this package.  It shares no code with the GPU library and imports nothing from it.
"""
