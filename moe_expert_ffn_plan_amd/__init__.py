"""MI355X-native fused MoE expert FFN: routing tables, grouped FP8 x FP4 GEMMs
with a fused SwiGLU/requant epilogue, and the top-k combine, as HIP kernels for
gfx950 behind a C ABI (``include/moe.h``).

The binding (``moe_expert_ffn_plan_amd.binding``) only marshals arguments;
it loads ``libmoe_mi355x.so`` from this directory and raises if it is
missing.  ``inputs`` draws seeded synthetic workloads.
"""
