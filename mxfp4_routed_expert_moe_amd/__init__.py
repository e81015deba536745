"""MI355X-native MXFP4 routed-expert MoE layer (DeepSeek-V4-Flash shape).

The compute path is the C-ABI library ``libmoe.so`` built from ``csrc/`` for
gfx950; ``binding`` marshals arguments to it.  ``workloads`` draws the seeded
synthetic inputs.
"""
