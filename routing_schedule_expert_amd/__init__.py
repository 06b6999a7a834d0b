"""MI355X-native share of a Mixture-of-Experts layer: on-device counting-sort
schedule, pull gather, SwiGLU grouped-GEMM expert FFN, fixed-order combine,
and the backward that reuses the same table.

The kernels are HIP for gfx950 behind the C ABI in ``include/moe.h``;
``routing_schedule_expert_amd.ops`` is the thin Python binding (argument
marshalling only, torch tensors for device memory and streams) and
``routing_schedule_expert_amd.inputs`` draws seeded synthetic inputs.
"""
