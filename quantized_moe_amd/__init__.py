"""MI355X-native routed-expert MoE layer with 2-bit block-quantized experts.

The compute lives in the HIP library libqmoe.so (C ABI: include/moe.h);
``quantized_moe_amd.lib`` is its thin Python binding and ``synth`` the
seeded synthetic-input generator.
"""
