"""MI355X (gfx950) MegaMoE expert pipeline for one rank: HIP kernels behind a C ABI.

`moe_expert_ffn_amd.megamoe` is the ctypes binding of include/megamoe.h,
`moe_expert_ffn_amd.inputs` draws the seeded synthetic workloads and
`moe_expert_ffn_amd.build` compiles libmegamoe.so with hipcc.
"""
