"""MI355X-native routed MoE layer served from an elastic GPU expert cache.

The compute path lives in the HIP/C++ library ``libft.so`` (C ABI declared in
``include/ft.h``); ``moe_expert_offload_amd.ft`` is its thin ctypes binding and
``moe_expert_offload_amd.synth`` holds the seeded synthetic input generators.
Importing this package loads nothing.
"""
